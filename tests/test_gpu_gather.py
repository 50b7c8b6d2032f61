"""GPU check of the same-index gather that prices the selected-token call
(sparse_gather_sum): its per-(row, kv head) sums of the selected K and V
rows' 32-bit words must equal numpy's exactly (integer sums mod 2^32, so the
order of the additions does not matter).  Padding, out-of-range entries,
lists longer than one table chunk (512 FP8 / 1,024 BF16 entries), short
batches (whose lists are split into pieces added atomically) and large ones
(one wave per whole list) are covered; non-selected pool slots are
NaN-poisoned, which changes the sums if any of them is read."""
import numpy as np
import pytest

import workloads as w

pytestmark = pytest.mark.gpu


def _expected(p) -> np.ndarray:
    """Word sums of every row's valid entries, per kv head (numpy, uint64 then mod 2^32)."""
    words_dtype = np.uint32
    k = np.ascontiguousarray(p.k_cache).view(words_dtype)
    v = np.ascontiguousarray(p.v_cache).view(words_dtype)
    seq = p.token_seq()
    T, hkv = p.num_tokens, p.num_kv_heads
    nw = k.shape[-1]
    out = np.zeros((T, hkv, nw), dtype=np.uint64)
    for t in range(T):
        b = seq[t]
        lk = p.seq_lens_k[b]
        sel = p.indices[t]
        sel = sel[(sel >= 0) & (sel < lk)]
        pages = p.block_table[b, sel // p.page_size]
        slots = sel % p.page_size
        if p.kv_layout == "NHD":
            rows = k[pages, slots].astype(np.uint64) + v[pages, slots].astype(np.uint64)  # [n, hkv, nw]
        else:
            rows = (k[pages, :, slots].astype(np.uint64) + v[pages, :, slots].astype(np.uint64))
        out[t] = rows.sum(0)
    return (out % (1 << 32)).astype(np.uint32)


CASES = [
    ("fp8_24to2", dict(seed=[101], lq=[20], lk=[3000], hq=24, hkv=2, n=700, kv=w.FP8, pad=0.0)),
    ("bf16_24to2_pad", dict(seed=[102], lq=[17], lk=[2500], hq=24, hkv=2, n=300, kv=w.BF16, pad=0.3)),
    ("fp8_long_lists", dict(seed=[103], lq=[5, 3], lk=[6000, 2200], hq=12, hkv=1, n=2100, kv=w.FP8, pad=0.1)),
    ("bf16_page64", dict(seed=[104], lq=[6], lk=[4000], hq=8, hkv=1, n=1030, kv=w.BF16, pad=0.0, page=64)),
    # more than 4,096 (row, kv head) jobs: no list pieces
    ("fp8_unsplit", dict(seed=[105], lq=[2100], lk=[3000], hq=24, hkv=2, n=300, kv=w.FP8, pad=0.1)),
    ("bf16_unsplit", dict(seed=[106], lq=[2050], lk=[2600], hq=24, hkv=2, n=530, kv=w.BF16, pad=0.0)),
]


@pytest.mark.parametrize("name,c", CASES, ids=[n for n, _ in CASES])
def test_gather_sum_exact(name, c):
    import torch

    import paged_gqa_attention_hd256_amd as pga
    from paged_gqa_attention_hd256_amd import problem_io

    p = w.make_sparse(name, c["seed"], c["lq"], c["lk"], c["hq"], c["hkv"], c["n"], kv_dtype=c["kv"],
                      page_size=c.get("page", 16), pad_fraction=c["pad"])
    p.indices[0, 1] = int(p.seq_lens_k[0]) + 5   # an entry past the context: skipped like padding
    p = w.poison_unused(p)
    print(f"case {name}", flush=True)
    dp = problem_io.to_device(p)
    got = pga.sparse_gather_sum(dp.cu_seqlens_q, dp.seq_lens_k, dp.indices, dp.kv)
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    exp = _expected(p)
    assert got.shape == exp.shape
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{name}: {len(bad)} sums differ, first at {bad[:3].tolist()}"


# ---------------------------------------------------------------------------
# The page-gather roof of the verify call (paged_attn_verify_gather_sum): per
# (sequence, kv head), the word sum of the K and V rows of every key below the
# history's length (none for a sequence without query tokens), exact.

def _expected_verify(p, max_kv_len) -> np.ndarray:
    k = np.ascontiguousarray(p.k_cache).view(np.uint32)
    v = np.ascontiguousarray(p.v_cache).view(np.uint32)
    lq = np.diff(p.cu_seqlens_q)
    out = np.zeros((len(p.seq_lens_k), p.num_kv_heads), dtype=np.uint64)
    for b, lk in enumerate(p.seq_lens_k):
        lk = min(int(lk), max_kv_len)
        if lq[b] <= 0 or lk <= 0:
            continue
        j = np.arange(lk)
        pages = p.block_table[b, j // p.page_size]
        slots = j % p.page_size
        if p.kv_layout == "NHD":
            rows = k[pages, slots].astype(np.uint64) + v[pages, slots].astype(np.uint64)  # [n, hkv, nw]
        else:
            rows = k[pages, :, slots].astype(np.uint64) + v[pages, :, slots].astype(np.uint64)
        out[b] = rows.sum(axis=(0, 2))
    return (out % (1 << 32)).astype(np.uint32)


VERIFY_CASES = [
    ("fp8_16to1", dict(seed=[111], lq=[4, 4, 2, 3], lk=[700, 65, 1500, 2049], hq=16, hkv=1, kv=w.FP8)),
    ("bf16_32to2", dict(seed=[112], lq=[3, 3], lk=[513, 1300], hq=32, hkv=2, kv=w.BF16)),
    ("fp8_hnd_page64", dict(seed=[113], lq=[2, 1], lk=[901, 64], hq=16, hkv=2, kv=w.FP8, layout="HND", page=64)),
    ("fp8_zero_q_tokens", dict(seed=[114], lq=[2, 0, 3], lk=[100, 50, 300], hq=16, hkv=1, kv=w.FP8)),
]


@pytest.mark.parametrize("name,c", VERIFY_CASES, ids=[n for n, _ in VERIFY_CASES])
@pytest.mark.parametrize("plan", ["exact_bound", "planned_64", "planned_0"])
def test_verify_gather_sum_exact(name, c, plan):
    import torch

    import paged_gqa_attention_hd256_amd as pga
    from paged_gqa_attention_hd256_amd import problem_io

    p = w.make_causal(name, c["seed"], c["lq"], c["lk"], c["hq"], c["hkv"], kv_dtype=c["kv"],
                      page_size=c.get("page", 16), layout=c.get("layout", "NHD"), mode="verify")
    p = w.poison_unused(p)
    mk = int(np.max(p.seq_lens_k)) if plan == "exact_bound" else 64 * 65  # past 64 tiles: the planned split
    split = 64 if plan == "planned_64" else 0
    print(f"case {name} {plan}", flush=True)
    dp = problem_io.to_device(p, max_kv_len=mk)
    got = pga.verify_gather_sum(dp.cu_seqlens_q, dp.seq_lens_k, max(1, int(np.diff(p.cu_seqlens_q).max())), mk,
                                dp.kv, kv_split_tokens=split)
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    exp = _expected_verify(p, mk)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{name}/{plan}: {len(bad)} sums differ, first at {bad[:3].tolist()}"
