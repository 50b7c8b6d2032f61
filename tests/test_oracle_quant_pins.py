"""Pins of the oracle's FP8 quantisation (CPU only).

The oracle encodes fp32 values to OCP E4M3FN by a nearest-value search over
its own decoded code table and quantises bf16 tensors per tensor.  Each test
below checks it against something other than itself: torch's own
``float8_e4m3fn`` conversion, numpy's IEEE fp32 division, closed forms
(round trips, midpoints, saturation, the largest element landing on 448) and
independent numpy page addressing for the key/value write.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as w

FINITE_POS = list(range(0x7F))  # 0x00 .. 0x7E: the finite non-negative codes, increasing


def _e4m3_value(code: int) -> float:
    return float(torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)[0])


def _torch_codes(y: np.ndarray) -> np.ndarray:
    """torch's RNE conversion of fp32 values already inside [-448, 448]."""
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _all_bf16_finite() -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits[np.isfinite(f)]


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_encoder_round_trips_every_finite_code():
    for c in FINITE_POS:
        for code in (c, c | 0x80):
            assert oracle.encode_e4m3fn(_e4m3_value(code)) == code, hex(code)


def test_encoder_ties_go_to_the_even_code_and_neighbours_to_the_nearer():
    for c in FINITE_POS[:-1]:
        lo, hi = _e4m3_value(c), _e4m3_value(c + 1)
        mid = np.float32((lo + hi) / 2)            # exact: both are short dyadic numbers
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode_e4m3fn(mid) == even
        assert oracle.encode_e4m3fn(-mid) == even | 0x80
        assert oracle.encode_e4m3fn(np.nextafter(mid, np.float32(0))) == c
        assert oracle.encode_e4m3fn(np.nextafter(mid, np.float32(np.inf))) == c + 1


def test_encoder_saturates_and_keeps_nan():
    big = np.float32(3.0e38)
    for y in (448.0, 449.0, 463.9, 464.0, 480.0, 1.0e6, float(big), float("inf")):
        assert oracle.encode_e4m3fn(y) == 0x7E
        assert oracle.encode_e4m3fn(-y) == 0xFE
    assert oracle.encode_e4m3fn(float("nan")) in (0x7F, 0xFF)
    assert oracle.encode_e4m3fn(0.0) == 0x00 and oracle.encode_e4m3fn(-0.0) == 0x80
    # below half the smallest subnormal (2^-10) everything rounds to a signed zero
    assert oracle.encode_e4m3fn(2.0 ** -10) == 0x00 and oracle.encode_e4m3fn(-(2.0 ** -11)) == 0x80
    assert oracle.encode_e4m3fn(2.0 ** -10 * 1.0001) == 0x01


@pytest.mark.parametrize("descale", [1.0, 2.0 ** -3, 0.37, 5.5e-3, 2.0 ** 6])
def test_quantiser_equals_numpy_division_then_torch_rne(descale):
    """Every finite bf16 pattern, quantised with a static descale: the oracle
    equals numpy's fp32 division followed by torch's conversion (clamped first,
    since torch does not saturate)."""
    bits = _all_bf16_finite()
    codes, used = oracle.quantize_fp8(bits, descale=descale)
    assert used == np.float32(descale)
    with np.errstate(over="ignore"):
        y = _bf16_to_f32(bits) / np.float32(descale)
    ref = _torch_codes(np.clip(y, -448.0, 448.0))
    np.testing.assert_array_equal(codes, ref)


def test_dynamic_scale_is_amax_over_448_and_largest_element_maps_to_448():
    rng = np.random.default_rng(3)
    for sigma in (1.0, 1e-3, 37.0):
        x = (rng.standard_normal(50_000) * sigma).astype(np.float32)
        bits = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
        codes, descale = oracle.quantize_fp8(bits)
        xf = _bf16_to_f32(bits)
        amax = np.max(np.abs(xf))
        assert np.float32(descale) == np.float32(amax) / np.float32(448.0)
        i = int(np.argmax(np.abs(xf)))
        assert codes[i] == (0xFE if xf[i] < 0 else 0x7E)
        ref = _torch_codes(np.clip(xf / np.float32(descale), -448.0, 448.0))
        np.testing.assert_array_equal(codes, ref)
        # dequantised values sit within half an E4M3 step (relative 2^-4) of x, or
        # within half the subnormal step 2^-10 in scaled units
        deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * descale
        tol = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * descale) * 1.0000001
        assert np.all(np.abs(deq - xf) <= tol)


def test_power_of_two_descale_hits_exact_ties():
    """With descale 2^-4 every y = x * 16 is exact, so bf16 inputs land on
    E4M3 midpoints; those must go to the even code."""
    bits = _all_bf16_finite()
    with np.errstate(over="ignore"):
        y = _bf16_to_f32(bits) * np.float32(16.0)
    sel = np.abs(y) <= 448.0
    codes, _ = oracle.quantize_fp8(bits[sel], descale=2.0 ** -4)
    np.testing.assert_array_equal(codes, _torch_codes(y[sel]))
    # at least some inputs are exact midpoints between two codes
    lo = _torch_codes(y[sel])
    n_ties = 0
    for c in range(0, 0x7E, 7):
        mid = np.float32((_e4m3_value(c) + _e4m3_value(c + 1)) / 2)
        n_ties += int(np.sum(y[sel] == mid))
    assert n_ties > 0 and lo.size > 0


def test_zero_tensor_uses_descale_one():
    codes, descale = oracle.quantize_fp8(np.array([0x0000, 0x8000, 0x0000], dtype=np.uint16))
    assert descale == 1.0
    assert list(codes) == [0x00, 0x80, 0x00]


def test_nan_elements_are_ignored_by_amax_and_stay_nan():
    bits = np.array([0x3F80, 0x7FC0, 0xC000], dtype=np.uint16)  # 1, NaN, -2
    codes, descale = oracle.quantize_fp8(bits)
    assert np.float32(descale) == np.float32(2.0) / np.float32(448.0)
    assert codes[1] in (0x7F, 0xFF) and codes[2] == 0xFE


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_new_keys_and_values_land_at_their_logical_positions(layout):
    p = w.make_prefill_quant("qw", [11, 0 if layout == "NHD" else 1], [5, 0, 19], [40, 3, 19], 8, 2,
                             layout=layout)
    k0, v0 = p.k_cache.copy(), p.v_cache.copy()
    oracle.write_new_kv(p, p.meta["k_new"], p.meta["v_new"], p.meta["cu_seqlens_k"])
    k_exp, v_exp = k0.copy(), v0.copy()
    P = p.page_size
    for b in range(p.num_seqs):
        q0, q1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        lk = int(p.seq_lens_k[b])
        for t in range(q1 - q0):
            pos = lk - (q1 - q0) + t
            page, slot = p.block_table[b, pos // P], pos % P
            for g in range(p.num_kv_heads):
                for new, exp, ds in ((p.meta["k_new"], k_exp, p.k_descale), (p.meta["v_new"], v_exp, p.v_descale)):
                    y = _bf16_to_f32(new[q0 + t, g]) / np.float32(ds)
                    row = _torch_codes(np.clip(y, -448.0, 448.0))
                    if layout == "NHD":
                        exp[page, slot, g] = row
                    else:
                        exp[page, g, slot] = row
    np.testing.assert_array_equal(p.k_cache, k_exp)
    np.testing.assert_array_equal(p.v_cache, v_exp)
    assert not np.any(p.k_cache == 0x7F) or np.array_equal(p.k_cache == 0x7F, k_exp == 0x7F)
