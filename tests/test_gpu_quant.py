"""GPU parity of the FP8 quantisation ahead of the prefill (through the C ABI).

Codes, descales and pool bytes are integer results: they must equal the
oracle's bit for bit (a NaN input may give either NaN code).  The quantised
prefill is then checked against the oracle's attention at the parity bar.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as w
from tests import gpu_util

pytestmark = pytest.mark.gpu

NAN_CODES = (0x7F, 0xFF)


def _bits_to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16)).view(torch.int16) \
        .view(torch.bfloat16).cuda()


def _assert_codes_equal(got: np.ndarray, ref: np.ndarray, what: str):
    got, ref = got.reshape(-1), ref.reshape(-1)
    nan_ref = np.isin(ref, NAN_CODES)
    assert np.array_equal(np.isin(got, NAN_CODES), nan_ref), f"{what}: NaN codes differ"
    bad = np.nonzero((got != ref) & ~nan_ref)[0]
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[:5]}: {got[bad[:5]]} vs {ref[bad[:5]]}"


def _quantize_q(bits: np.ndarray, descale=None):
    import torch
    import paged_gqa_attention_hd256_amd as pga

    q = _bits_to_dev(bits)
    ds = None if descale is None else torch.tensor([descale], dtype=torch.float32, device="cuda")
    codes, used = pga.prefill_quantize_fp8(q, q_descale=ds)
    torch.cuda.synchronize()
    return codes.view(torch.uint8).cpu().numpy(), float(used.cpu()[0])


def _all_patterns(finite_only: bool) -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if finite_only:
        f = (bits.astype(np.uint32) << 16).view(np.float32)
        bits = np.where(np.isfinite(f), bits, np.uint16(0))
    return bits.reshape(32, 8, 256)


@pytest.mark.parametrize("descale", [1.0, 2.0 ** -4, 0.37, 5.5e-3, 64.0, 2.0 ** -70, 1.0e30])
def test_every_bf16_pattern_with_a_given_descale(descale):
    """All 65,536 bf16 patterns (NaN and infinities included) against the
    oracle; 2^-4 puts inputs on exact E4M3 ties, 2^-70 and 1e30 take the plain
    division path."""
    bits = _all_patterns(finite_only=False)
    got, used = _quantize_q(bits, descale)
    ref, ref_ds = oracle.quantize_fp8(bits, descale=descale)
    assert used == ref_ds
    _assert_codes_equal(got, ref, f"descale {descale}")


def test_every_finite_bf16_pattern_with_the_dynamic_descale():
    bits = _all_patterns(finite_only=True)
    got, used = _quantize_q(bits)
    ref, ref_ds = oracle.quantize_fp8(bits)
    assert np.float32(used) == np.float32(ref_ds)
    _assert_codes_equal(got, ref, "dynamic, all finite patterns")


@pytest.mark.parametrize("T,hq,sigma", [(1, 8, 1.0), (37, 8, 3.0), (300, 16, 1e-3), (4097, 8, 1.0)])
def test_dynamic_descale_on_normal_draws(T, hq, sigma):
    rng = np.random.default_rng(T)
    x = (rng.standard_normal(T * hq * 256) * sigma).astype(np.float32)
    u = x.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16).reshape(T, hq, 256)
    got, used = _quantize_q(bits)
    ref, ref_ds = oracle.quantize_fp8(bits)
    assert np.float32(used) == np.float32(ref_ds)
    _assert_codes_equal(got, ref, f"T={T} hq={hq}")


def test_empty_query_gives_descale_one():
    got, used = _quantize_q(np.zeros((0, 8, 256), dtype=np.uint16))
    assert got.size == 0 and used == 1.0


QUANT_CASES = [
    ("one_seq_nhd", dict(lens_q=[70], lens_k=[300], hq=8, hkv=1)),
    ("three_seqs_two_heads", dict(lens_q=[5, 0, 19], lens_k=[40, 3, 19], hq=8, hkv=2)),
    ("hnd_page64", dict(lens_q=[33, 64], lens_k=[500, 64], hq=16, hkv=2, layout="HND", page_size=64)),
    ("r12_ragged", dict(lens_q=[1, 17, 130], lens_k=[1, 200, 1000], hq=24, hkv=2)),
]


def _quant_problem(name, c, seed):
    return w.make_prefill_quant(name, [seed, 0], c["lens_q"], c["lens_k"], c["hq"], c["hkv"],
                                layout=c.get("layout", "NHD"), page_size=c.get("page_size", 16))


def _gpu_quantize(p):
    import torch
    from paged_gqa_attention_hd256_amd import problem_io

    dp = problem_io.to_device(p)
    problem_io.run(dp, stage="quant")
    torch.cuda.synchronize()
    return (dp.quant.q_fp8.view(torch.uint8).cpu().numpy(), float(dp.quant.q_descale.cpu()[0]),
            dp.kv.k_cache.view(torch.uint8).cpu().numpy(), dp.kv.v_cache.view(torch.uint8).cpu().numpy())


@pytest.mark.parametrize("name,c", QUANT_CASES, ids=[n for n, _ in QUANT_CASES])
def test_quantize_q_and_new_keys_values_bit_exact(name, c):
    p = _quant_problem(name, c, 31)
    ref = oracle.quantized_problem(p)
    q_codes, ds, k_pool, v_pool = _gpu_quantize(p)
    assert np.float32(ds) == np.float32(ref.q_descale)
    _assert_codes_equal(q_codes, ref.q, f"{name} q")
    # the whole pool: new rows equal the oracle's, every other byte is untouched
    assert np.array_equal(k_pool, ref.k_cache), f"{name}: key pool differs"
    assert np.array_equal(v_pool, ref.v_cache), f"{name}: value pool differs"


@pytest.mark.parametrize("name,c", QUANT_CASES, ids=[n for n, _ in QUANT_CASES])
def test_quantized_prefill_parity(name, c):
    p = _quant_problem(name, c, 47)
    ref_p = oracle.quantized_problem(p)
    ref, ref_lse = oracle.attention(ref_p)
    got, got_lse = gpu_util.run_gpu(p)
    gpu_util.assert_parity(got, got_lse, ref, ref_lse, what=f"quantized prefill {name}")


def test_full_size_quantization_bit_exact():
    """The 16k-new / 32k-context quantising prefill, in the launch the
    benchmark times: every Q code, the descale and the whole pool."""
    p = w.config("prefill_quant_32k")
    ref = oracle.quantized_problem(p)
    q_codes, ds, k_pool, v_pool = _gpu_quantize(p)
    assert np.float32(ds) == np.float32(ref.q_descale)
    _assert_codes_equal(q_codes, ref.q, "prefill_quant_32k q")
    assert np.array_equal(k_pool, ref.k_cache) and np.array_equal(v_pool, ref.v_cache)
