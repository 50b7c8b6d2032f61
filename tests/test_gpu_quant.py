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


@pytest.mark.parametrize("T,hq,sigma", [(1, 8, 1.0), (37, 8, 3.0), (300, 16, 1e-3), (4096, 8, 1.0), (4097, 8, 1.0),
                                        (8193, 8, 0.5)])
def test_dynamic_descale_on_normal_draws(T, hq, sigma):
    rng = np.random.default_rng(T)
    x = (rng.standard_normal(T * hq * 256) * sigma).astype(np.float32)
    u = x.view(np.uint32)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16).reshape(T, hq, 256)
    got, used = _quantize_q(bits)
    ref, ref_ds = oracle.quantize_fp8(bits)
    assert np.float32(used) == np.float32(ref_ds)
    _assert_codes_equal(got, ref, f"T={T} hq={hq}")


def _resident_capacity_chunks() -> int:
    """16-byte Q chunks the single-read path holds: 16 per thread, 1,024
    threads per workgroup, one workgroup per CU."""
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count * 1024 * 16


def test_dynamic_descale_beyond_the_resident_capacity():
    """One token more than the registers hold: the two-launch path (Q read
    twice) must give the same codes and descale."""
    hq = 8
    T = _resident_capacity_chunks() // (hq * 32) + 1
    rng = np.random.default_rng(5)
    bits = (rng.standard_normal(T * hq * 256, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = bits.reshape(T, hq, 256)
    bits[T - 1, hq - 1, 255] = 0x4300  # the largest magnitude (128.0) in the very last chunk
    got, used = _quantize_q(bits)
    ref, ref_ds = oracle.quantize_fp8(bits)
    assert np.float32(used) == np.float32(ref_ds) == np.float32(128.0 / 448.0)
    _assert_codes_equal(got, ref, f"T={T} (two-launch path)")


def test_resident_path_barrier_slots_from_a_dirty_workspace():
    """The single-read path on a workspace full of stale bytes: every
    workgroup (one per CU) publishes its partial maximum under one tag per
    call, a new tag on the next call, the largest partial is the input's
    largest magnitude, and no wait expires (the flag word keeps its stale
    bytes)."""
    import torch
    import paged_gqa_attention_hd256_amd as pga

    T, hq = 4097, 8
    rng = np.random.default_rng(9)
    bits = (rng.standard_normal(T * hq * 256, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = bits.reshape(T, hq, 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ws = torch.full((pga.quantize_workspace_bytes(),), 0xAB, dtype=torch.uint8, device="cuda")
    ref, ref_ds = oracle.quantize_fp8(bits)
    tags = []
    for _ in range(2):
        codes, used = pga.prefill_quantize_fp8(_bits_to_dev(bits), workspace=ws)
        torch.cuda.synchronize()
        words = ws[4096:].view(torch.int64).cpu().numpy().view(np.uint64)
        slots = words[:1024 * 16:16]
        assert (slots[cus:] == np.uint64(0xABABABABABABABAB)).all(), "slots beyond the grid written"
        tag = slots[:cus] >> np.uint64(16)
        assert (tag == tag[0]).all() and int(tag[0]) & 1 == 1
        assert int((slots[:cus] & np.uint64(0xFFFF)).max()) == int((bits & 0x7FFF).max())
        assert words[1024 * 16] == np.uint64(0xABABABABABABABAB), "a barrier wait expired"
        tags.append(int(tag[0]))
        assert np.float32(float(used.cpu()[0])) == np.float32(ref_ds)
        _assert_codes_equal(codes.view(torch.uint8).cpu().numpy(), ref, "dirty workspace")
    assert tags[0] != tags[1]


def test_dynamic_descale_into_an_8_byte_aligned_output():
    """Codes written to an output that is 8- but not 16-byte aligned (the
    single-read path stores 16 bytes per lane, so the two-launch path runs)."""
    import torch
    import paged_gqa_attention_hd256_amd as pga

    T, hq = 300, 8
    rng = np.random.default_rng(3)
    bits = (rng.standard_normal(T * hq * 256, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = bits.reshape(T, hq, 256)
    n = T * hq * 256
    buf = torch.full((n + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    out = buf[8:8 + n].view(torch.float8_e4m3fn).view(T, hq, 256)
    assert out.data_ptr() % 16 == 8
    _, used = pga.prefill_quantize_fp8(_bits_to_dev(bits), q_fp8=out)
    torch.cuda.synchronize()
    ref, ref_ds = oracle.quantize_fp8(bits)
    assert np.float32(float(used.cpu()[0])) == np.float32(ref_ds)
    host = buf.cpu().numpy()
    _assert_codes_equal(host[8:8 + n], ref, "8-byte aligned output")
    assert (host[:8] == 0x5A).all() and (host[8 + n:] == 0x5A).all(), "bytes outside the output changed"


@pytest.mark.parametrize("amax", [2.0 ** -126, 1e-30, 3.0e-5, 0.37, 1.0, 448.0, 1.0e10, 3.0e38])
def test_dynamic_descale_every_pattern_up_to_amax(amax):
    """Every finite bf16 pattern of magnitude up to amax (amax itself
    included, NaNs sprinkled in) under the dynamic descale amax / 448: the
    quotients reach 448 (1 + 2^-23) at x = amax, and the descales span both
    division paths (2^-126 / 448 and 3e38 / 448 lie outside the reciprocal's
    range)."""
    cap = int(np.array([amax], dtype=np.float32).view(np.uint32)[0] >> 16)
    mags = np.arange(cap + 1, dtype=np.uint32)
    bits = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    bits[::997] = 0x7FC1  # NaNs, left out of amax
    bits[1] = np.uint16(cap)
    pad = (-bits.size) % (8 * 256)
    bits = np.concatenate([bits, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 8, 256)
    got, used = _quantize_q(bits)
    ref, ref_ds = oracle.quantize_fp8(bits)
    assert np.float32(used) == np.float32(ref_ds)
    _assert_codes_equal(got, ref, f"amax {amax}")


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
