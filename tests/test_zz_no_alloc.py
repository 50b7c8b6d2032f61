"""The allocation-free verify entry point (paged_attn_verify_noalloc) against
paged_attn_verify with a caller workspace: the same kernels, so the outputs
must agree bit for bit, and both must meet the parity bar against the fp64
oracle.  Two calls in a row share the library's fixed scratch: the second is
smaller and uses the other partial width (BF16 V after FP8 V), so whatever
the first call left in the scratch must not leak into it.
"""
import numpy as np
import pytest

import oracle
import workloads as w
from tests.gpu_util import LSE_MARGIN, LSE_SENTINEL, OUT_MARGIN, OUT_SENTINEL, Guarded, assert_parity

pytestmark = pytest.mark.gpu


def _problems():
    big = w.make_causal("noalloc_fp8", [91], [4] * 12, [6000, 65, 4100, 2500, 777, 3333, 5999, 129, 1024, 4, 2048,
                                                      3001], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5, mode="verify")
    small = w.make_causal("noalloc_bf16", [92], [3, 1, 2], [900, 1500, 64], 12, 2, kv_dtype=w.BF16, mode="verify")
    return [(w.poison_unused(big), 256), (w.poison_unused(small), 64)]


def test_noalloc_matches_workspace_entry_point_two_calls():
    import torch

    import paged_gqa_attention_hd256_amd as pga
    from paged_gqa_attention_hd256_amd import problem_io

    for p, split in _problems():
        print(f"case {p.name} split={split}", flush=True)
        ref, ref_lse = oracle.attention(p)
        dp = problem_io.to_device(p, kv_split_tokens=split)
        assert dp.workspace is not None  # the workspace call does split the histories
        # the existing entry point, with the caller's workspace
        problem_io.run(dp)
        torch.cuda.synchronize()
        ws_bits = dp.out.view(torch.int16).cpu().numpy().copy()
        ws_lse = dp.lse.cpu().numpy().copy()
        # the allocation-free entry point, into guarded buffers
        g_out = Guarded(dp.out.numel(), torch.bfloat16, OUT_MARGIN, OUT_SENTINEL)
        g_lse = Guarded(dp.lse.numel(), torch.float32, LSE_MARGIN, LSE_SENTINEL)
        out = g_out.view.view(dp.out.shape)
        lse = g_lse.view.view(dp.lse.shape)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        pga.paged_attn_verify_noalloc(dp.q, dp.cu_seqlens_q, dp.seq_lens_k, dp.max_q_len, dp.max_kv_len, dp.kv,
                                      dp.softmax_scale, out, kv_split_tokens=dp.kv_split_tokens, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        g_out.check(f"{p.name}: out")
        g_lse.check(f"{p.name}: lse")
        bits = out.view(torch.int16).cpu().numpy()
        got_lse = lse.cpu().numpy()
        assert np.array_equal(bits, ws_bits), f"{p.name}: output differs from the workspace call"
        assert np.array_equal(got_lse, ws_lse), f"{p.name}: lse differs from the workspace call"
        assert_parity(bits, got_lse, ref, ref_lse, what=f"{p.name}/noalloc")
