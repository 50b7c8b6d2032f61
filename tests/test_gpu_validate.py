"""GPU checks of pga_validate_inputs (through the C ABI).

Valid workloads report no violation; copies with one planted defect (made on
the host, seen only by the validation kernels, which read inside the extents
the host arguments give) report exactly that defect."""
from __future__ import annotations

import numpy as np
import pytest

import workloads as w

pytestmark = pytest.mark.gpu

INVALID = 7


def _dev(p):
    from paged_gqa_attention_hd256_amd import problem_io
    return problem_io.to_device(p)


def _validate(dp, lens=True, **kw):
    import paged_gqa_attention_hd256_amd as pga

    if lens:
        kw.setdefault("seq_lens_k", dp.seq_lens_k)
    else:
        kw.setdefault("cu_seqlens_k", dp.cu_seqlens_k)
    return pga.validate_inputs(dp.cu_seqlens_q, dp.kv, **kw)


def _problems():
    yield w.config("tiny_verify")
    yield w.make_causal("v_multi", [91, 0], [4, 1, 3], [70, 1, 300], 16, 1, kv_dtype=w.FP8, mode="verify")
    yield w.make_causal("pf", [91, 1], [40, 9], [170, 9], 8, 1, kv_dtype=w.FP8, q_dtype=w.FP8, mode="prefill")
    yield w.make_sparse("sp", [91, 2], [6, 3], [900, 50], 24, 2, 100, kv_dtype=w.FP8, pad_fraction=0.25)


@pytest.mark.parametrize("p", list(_problems()), ids=lambda p: p.name)
def test_valid_inputs_report_nothing(p):
    dp = _dev(p)
    idx = dp.indices
    st, counts = _validate(dp, lens=p.mode != "prefill", max_q_len=dp.max_q_len, max_kv_len=dp.max_kv_len,
                           indices=idx)
    assert st == 0 and counts == [0, 0, 0, 0], counts


def test_planted_defects_are_counted():
    import torch

    p = w.make_causal("v_multi", [92, 0], [4, 1, 3], [70, 1, 300], 16, 1, kv_dtype=w.FP8, mode="verify")
    dp = _dev(p)
    bt0, lk0 = dp.kv.block_table.clone(), dp.seq_lens_k.clone()

    # one block-table entry of a visible key outside the pool, one negative
    dp.kv.block_table[0, 2] = p.num_pages
    dp.kv.block_table[2, 18] = -1
    st, counts = _validate(dp)
    assert st == INVALID and counts == [0, 0, 2, 0], counts
    # an entry past the last key of its sequence is padding, not a defect
    dp.kv.block_table.copy_(bt0)
    dp.kv.block_table[0, 5] = -7                      # Lk = 70 uses columns 0..4
    st, counts = _validate(dp)
    assert st == 0 and counts == [0, 0, 0, 0], counts

    # Lk < Lq for one sequence
    dp.kv.block_table.copy_(bt0)
    dp.seq_lens_k[1] = 0
    st, counts = _validate(dp)
    assert st == INVALID and counts[0] == 1, counts
    # lengths beyond the host bounds the caller would pass
    dp.seq_lens_k.copy_(lk0)
    st, counts = _validate(dp, max_q_len=3, max_kv_len=299)
    assert st == INVALID and counts[1] == 2, counts   # Lq 4 > 3 and Lk 300 > 299
    # a history longer than the block-table row: counted, and no read past the row
    dp.seq_lens_k[2] = 16 * p.block_table.shape[1] + 1
    st, counts = _validate(dp)
    assert st == INVALID and counts[1] == 1, counts
    torch.cuda.synchronize()


def test_index_entries_past_the_context_are_reported_not_failed():
    p = w.make_sparse("sp", [93, 0], [5], [400], 24, 2, 64, kv_dtype=w.FP8)
    dp = _dev(p)
    dp.indices[1, 3] = 400          # == Lk
    dp.indices[4, 0] = 1 << 20
    st, counts = _validate(dp, indices=dp.indices)
    assert st == 0 and counts == [0, 0, 0, 2], counts


def test_token_count_mismatch_is_a_length_defect():
    import paged_gqa_attention_hd256_amd as pga

    p = w.make_sparse("sp", [94, 0], [5, 2], [400, 30], 24, 2, 16, kv_dtype=w.FP8)
    dp = _dev(p)
    short = dp.indices[:6].contiguous()       # 6 rows given, cu_seqlens_q says 7
    st, counts = pga.validate_inputs(dp.cu_seqlens_q, dp.kv, seq_lens_k=dp.seq_lens_k, indices=short)
    assert st == INVALID and counts[0] == 1, counts
    assert np.all(np.asarray(counts[1:3]) == 0)
