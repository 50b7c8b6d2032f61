"""Pins of the fp64 oracle against things other than itself.

Each test fixes part of the definition the oracle writes out:
* codecs against torch's own float8_e4m3fn / bfloat16 conversions;
* the whole result against torch's fp64 scaled_dot_product_attention on
  contiguous keys with a library-built (torch.tril) bottom-right causal mask;
* page addressing by permutation and layout invariance;
* normalisation, the lse, the visible set and one-key outputs exactly;
* closed forms (q = 0, constant V, descale algebra);
* the sparse variant against dense attention with the unselected keys masked;
* the log-sum-exp merge identity used by split-KV.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as w
from tests import refs


# ---------------------------------------------------------------- codecs ---
def test_e4m3fn_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3fn(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_bf16_decoder_matches_torch():
    rng = np.random.Generator(np.random.PCG64(7))
    bits = np.concatenate([rng.integers(0, 1 << 16, 4000, dtype=np.uint32).astype(np.uint16),
                           np.array([0, 0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80, 0x7F80], dtype=np.uint16)])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_generator_bf16_rounding_is_rne():
    # The generator's bf16 encoder must agree with torch's RNE conversion.
    x = np.random.Generator(np.random.PCG64(3)).standard_normal(100000).astype(np.float32)
    x[:4] = np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39], dtype=np.float32)  # ties + subnormal
    ours = w.synth._to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------- dense reference ---
def _small_cases():
    yield w.make_causal("bf16_verify", [101], [2, 3, 1], [37, 64, 17], 16, 1, kv_dtype=w.BF16)
    yield w.make_causal("fp8_verify", [102], [4, 4], [50, 129], 32, 2, kv_dtype=w.FP8, kv_sigma=0.5)
    yield w.make_causal("fp8_prefill", [103], [24, 9], [40, 9], 8, 1, kv_dtype=w.FP8, q_dtype=w.FP8,
                        mode="prefill")
    yield w.make_causal("hnd_layout", [104], [3, 2], [33, 47], 12, 2, kv_dtype=w.BF16, layout="HND")
    yield w.make_causal("page64", [105], [2, 4], [70, 130], 16, 1, kv_dtype=w.FP8, page_size=64)


@pytest.mark.parametrize("case", list(_small_cases()), ids=lambda p: p.name)
def test_oracle_equals_sdpa_on_contiguous_keys(case):
    out, lse = oracle.attention(case)
    ref = refs.dense_attention(case)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert refs.max_abs(out, ref) <= 1e-12 * max(1.0, np.abs(ref).max())
    assert refs.rel_l2(out, ref) < 1e-13


def test_page_permutation_and_layout_invariance_bitwise():
    p = w.make_causal("perm", [111], [2, 4, 1], [33, 48, 15 + 16 * 3], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    base, base_lse = oracle.attention(p)
    for seed, layout in ((1, "NHD"), (2, "HND"), (3, "NHD")):
        q = refs.repack(p, seed, layout, extra_pages=5, fill_code=w.NAN_CODE[p.kv_dtype])
        out, lse = oracle.attention(q)
        assert np.array_equal(out, base) and np.array_equal(lse, base_lse)


@pytest.mark.parametrize("tail", [1, 8, 15, 0])
def test_ragged_last_page_matches_sdpa(tail):
    lk = 16 * 4 + tail
    p = w.make_causal("tail", [120, tail], [3], [lk], 16, 1, kv_dtype=w.BF16)
    w.poison_unused(p)  # NaN in every slot past lk: a read of one would show
    out, _ = oracle.attention(p)
    ref = refs.dense_attention(p)
    assert np.all(np.isfinite(out))
    assert refs.rel_l2(out, ref) < 1e-13


# ------------------------------------------------------- causal rule ---
def test_bottom_right_causal_visible_sets_by_enumeration():
    """For every Lq in 1..6 and Lk in Lq..Lq+7, the keys each query sees (the
    support of its weights) equal the set enumerated from "new tokens are the last
    Lq positions of the sequence and see no later position", and the output equals
    SDPA with torch.tril's mask."""
    for lq in range(1, 7):
        for lk in range(lq, lq + 8):
            p = w.make_causal("bf", [130, lq, lk], [lq], [lk], 2, 1, kv_dtype=w.BF16, page_size=4)
            positions = list(range(lk))[lk - lq:]  # absolute positions of the new tokens
            for t in range(lq):
                expect = {j for j in range(lk) if j <= positions[t]}
                for h in range(2):
                    probs = oracle.causal_probs(p, t, h)
                    assert set(np.nonzero(probs)[0].tolist()) == expect
            out, _ = oracle.attention(p)
            assert refs.rel_l2(out, refs.dense_attention(p)) < 1e-13


def test_weights_sum_to_one_and_lse_consistent():
    p = w.make_causal("norm", [140], [3, 2], [41, 70], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    out, lse = oracle.attention(p)
    q = refs.decode_torch(p.q, p.q_dtype).numpy() * p.q_descale
    for tok in range(p.num_tokens):
        b = int(np.searchsorted(p.cu_seqlens_q, tok, side="right") - 1)
        k, v = refs.logical_kv(p, b)
        for h in (0, 7, 15):
            probs = oracle.causal_probs(p, tok, h)
            vis = probs > 0
            assert abs(probs.sum() - 1.0) < 1e-13
            assert np.all(probs[vis] <= 1.0)
            # lse pins the scores: p_j = exp(s_j - lse) with s_j computed here.
            s = p.softmax_scale * (k[:, 0, :].numpy() @ q[tok, h])
            np.testing.assert_allclose(np.exp(s[vis] - lse[tok, h]), probs[vis], rtol=1e-12, atol=0)
            # and the output is the probability-weighted sum of V rows.
            np.testing.assert_allclose(out[tok, h], probs @ v[:, 0, :].numpy(), rtol=1e-12, atol=1e-15)


def test_one_visible_key_gives_v_exactly():
    # Prefill with Lk == Lq: token 0 sees only key 0.
    p = w.make_causal("one", [150], [5], [5], 8, 1, kv_dtype=w.FP8, q_dtype=w.FP8, mode="prefill")
    out, lse = oracle.attention(p)
    _, v = refs.logical_kv(p, 0)
    for h in range(8):
        assert np.array_equal(out[0, h], v[0, 0].numpy())
    # Sparse row with a single index.
    s = w.make_sparse("one_sp", [151], [3], [40], 24, 2, 1, kv_dtype=w.BF16)
    out, _ = oracle.attention(s)
    _, v = refs.logical_kv(s, 0)
    for t in range(3):
        j = s.indices[t, 0]
        for h in range(24):
            assert np.array_equal(out[t, h], v[j, h // 12].numpy())


# ------------------------------------------------------- closed forms ---
def test_zero_query_gives_mean_of_visible_values():
    p = w.make_causal("q0", [160], [2, 3], [20, 35], 16, 1, kv_dtype=w.BF16)
    p.q[:] = 0
    out, lse = oracle.attention(p)
    for b in range(p.num_seqs):
        _, v = refs.logical_kv(p, b)
        lq, lk = int(p.q_lens[b]), int(p.seq_lens_k[b])
        for t in range(lq):
            tok = int(p.cu_seqlens_q[b]) + t
            n = lk - lq + t + 1
            np.testing.assert_allclose(out[tok], np.broadcast_to(v[:n, 0].numpy().mean(0), (16, 256)),
                                       rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[tok], np.log(n), rtol=1e-14)


def test_constant_values_and_descale_algebra():
    p = w.make_causal("cv", [170], [4], [52], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    base, base_lse = oracle.attention(p)
    c = w.make_causal("cv", [170], [4], [52], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    c.v_cache[:] = 0x40  # every V element is 2.0
    out, _ = oracle.attention(c)
    np.testing.assert_allclose(out, 2.0 * c.v_descale, rtol=1e-14)
    # v_descale x2 doubles the output exactly.
    d = w.make_causal("cv", [170], [4], [52], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    d.v_descale = p.v_descale * 2
    out, lse = oracle.attention(d)
    assert np.array_equal(out, 2 * base) and np.array_equal(lse, base_lse)
    # k_descale x2 with softmax_scale / 2 leaves the result unchanged.
    e = w.make_causal("cv", [170], [4], [52], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    e.k_descale, e.softmax_scale = p.k_descale * 2, p.softmax_scale / 2
    out, lse = oracle.attention(e)
    np.testing.assert_allclose(out, base, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(lse, base_lse, rtol=1e-14)


# ------------------------------------------------------------ sparse ---
@pytest.mark.parametrize("kv_dtype", [w.BF16, w.FP8])
def test_sparse_equals_dense_with_unselected_keys_masked(kv_dtype):
    s = w.make_sparse("sp", [180], [5, 3], [90, 200], 24, 2, 37, kv_dtype=kv_dtype, width=40)
    out, lse = oracle.attention(s)
    ref = refs.dense_attention(s, refs.sparse_mask_of(s))
    assert np.all(np.isfinite(out))
    assert refs.rel_l2(out, ref) < 1e-13


def test_sparse_padding_entries_are_skipped():
    s = w.make_sparse("pad", [181], [6], [300], 24, 2, 50, kv_dtype=w.BF16, width=64, pad_fraction=0.2)
    out, _ = oracle.attention(s)
    # Entries >= Lk are padding too: replace every -1 by Lk or a large value.
    t = w.make_sparse("pad", [181], [6], [300], 24, 2, 50, kv_dtype=w.BF16, width=64, pad_fraction=0.2)
    t.indices[t.indices < 0] = 300 + np.arange((t.indices < 0).sum()) % 7 * 1000
    out2, _ = oracle.attention(t)
    assert np.array_equal(out, out2)
    # An all-padding row: out = 0, lse = -inf.
    t.indices[2, :] = -1
    out3, lse3 = oracle.attention(t)
    assert np.all(out3[2] == 0) and np.all(np.isneginf(lse3[2]))


# ---------------------------------------------------------- LSE merge ---
def test_lse_merge_of_key_segments_equals_whole():
    """Attention over disjoint key segments, merged by log-sum-exp weights,
    equals attention over their union; an empty segment has weight 0."""
    p = w.make_causal("merge", [190], [3], [150], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
    whole, whole_lse = oracle.attention(p)
    lq, lk = 3, 150
    seg = 64
    outs, lses = [], []
    for lo in range(0, lk + seg, seg):  # the last segment is empty
        s = w.make_causal("merge", [190], [3], [150], 16, 1, kv_dtype=w.FP8, kv_sigma=0.5)
        idx = np.full((lq, seg), -1, dtype=np.int32)
        for t in range(lq):
            last = lk - lq + t
            keys = [j for j in range(lo, lo + seg) if j <= last]
            idx[t, :len(keys)] = keys
        s.mode, s.indices = "sparse", idx
        o, l = oracle.attention(s)
        outs.append(o)
        lses.append(l)
    L = np.stack(lses)                     # [S, T, H]
    O = np.stack(outs)                     # [S, T, H, D]
    assert np.all(np.isneginf(L[-1])) and np.all(O[-1] == 0)
    M = L.max(0)
    wts = np.where(np.isneginf(L), 0.0, np.exp(L - M))
    merged = (wts[..., None] * O).sum(0) / wts.sum(0)[..., None]
    np.testing.assert_allclose(merged, whole, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(M + np.log(wts.sum(0)), whole_lse, rtol=1e-13)


# ------------------------------------------------- workload accounting ---
def test_visible_pairs_and_flop_counts_of_prefill_workloads():
    # 16384 new tokens after 16384 / 114688 cached: per-head visible pairs and the
    # 4 * 256 flops per (pair, head) give 3.2986 and 16.493 TFLOP per call.
    for lk, tflop in ((32768, 3.2986), (131072, 16.493)):
        p = w.make_causal("acct", [1], [4], [8], 8, 1)  # shape holder only
        p.cu_seqlens_q = np.array([0, 16384], dtype=np.int32)
        p.seq_lens_k = np.array([lk], dtype=np.int32)
        pairs = w.visible_pairs(p)
        assert pairs == 16384 * (lk - 16384) + 16384 * 16385 // 2
        assert abs(4 * 256 * 8 * pairs / 1e12 - tflop) < 5e-4
