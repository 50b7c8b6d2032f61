"""Seeded random shapes for all three calls, against the fp64 oracle.

Each case draws its configuration from its own seed: batch size and ragged
lengths, GQA ratio (1:1 up to 32:1) and kv heads, q_len (verify), query and
KV encodings, page size 16 ... 256 and both pool layouts, the verify split
setting, the sparse list width and padding, the softmax scale and the input
spread (K/V up to 1, queries up to 3: peaked softmaxes and scores far from
zero included).  Every pool slot outside the visible keys is NaN-poisoned, and
outputs sit inside guard margins (run_gpu), so nothing may be written outside
the outputs.  The shapes stay inside each call's documented envelope (verify:
r * max q_len <= 64 rows per kv group; prefill: FP8 queries only with FP8
keys).

Bars, scaled where these shapes leave the benchmarked value ranges:
- every output element within 1e-2 of the oracle beyond its own bf16
  rounding (a peaked softmax returns nearly one V row, |out| up to ~5, where
  half a bf16 step is already 0.0156), and rel-L2 <= 2e-3;
- lse within 1e-3 + 5e-5 |lse|: the scaled FP8 matrix instruction drops,
  within each group of eight products, those more than 2^16 below the
  group's largest (probed on the part: 2^16 + 7 x 1 sums to 2^16), so score
  errors grow with the scores' size; at |lse| ~ 40 they reach ~1e-3, while
  the outputs stay at the bf16 floor.
"""
import numpy as np
import pytest

import oracle
import workloads as w
from tests import refs
from tests.gpu_util import bf16_bits_to_f64, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 36


def _draw(i):
    rng = np.random.default_rng([2024, i])
    mode = ("verify", "prefill", "sparse")[i % 3]
    hkv = int(rng.choice([1, 2]))
    page = int(rng.choice([16, 16, 32, 64, 128, 256]))
    layout = str(rng.choice(["NHD", "HND"]))
    kv = w.FP8 if rng.random() < 0.6 else w.BF16
    scale = float(rng.choice([1.0 / 16.0, 1.0 / 8.0, 0.3]))
    # K/V spread up to 1 (the absolute bar of 1e-2 is stated for outputs of
    # that scale: bf16 rounding of |out| ~ 8 alone exceeds it); peaked
    # softmaxes come from the query spread and the scale instead.
    sigma = float(rng.choice([0.5, 1.0]))
    q_sigma = float(rng.choice([0.5, 1.0, 2.0, 3.0]))
    B = int(rng.integers(1, 5))
    c = dict(mode=mode, hkv=hkv, page=page, layout=layout, kv=kv, scale=scale, sigma=sigma, q_sigma=q_sigma)
    if mode == "verify":
        lq = rng.integers(1, 5, size=B)
        r = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
        r = min(r, 64 // int(lq.max()))
        lk = lq + rng.integers(0, 2500, size=B)
        c.update(lq=lq.tolist(), lk=lk.tolist(), hq=r * hkv, q=w.BF16,
                 split=[None, 64, 128, 256, 1024][int(rng.integers(0, 5))])
    elif mode == "prefill":
        lq = rng.integers(1, 160, size=B)
        lk = lq + rng.integers(0, 700, size=B)
        r = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        q = w.FP8 if (kv == w.FP8 and rng.random() < 0.7) else w.BF16
        c.update(lq=lq.tolist(), lk=lk.tolist(), hq=r * hkv, q=q)
    else:
        lq = rng.integers(1, 12, size=B)
        lk = lq + rng.integers(0, 3000, size=B)
        r = int(rng.choice([1, 3, 6, 8, 12, 16, 24, 32]))
        n = int(rng.integers(1, 1300))
        c.update(lq=lq.tolist(), lk=lk.tolist(), hq=r * hkv, n=n, pad=float(rng.choice([0.0, 0.0, 0.3])),
                 width=n + int(rng.integers(0, 40)))
    return c


def _problem(i, c):
    name = f"rand{i}_{c['mode']}"
    if c["mode"] == "sparse":
        return w.make_sparse(name, [3100, i], c["lq"], c["lk"], c["hq"], c["hkv"], c["n"], kv_dtype=c["kv"],
                             page_size=c["page"], layout=c["layout"], kv_sigma=c["sigma"],
                             softmax_scale=c["scale"], width=c["width"], pad_fraction=c["pad"])
    return w.make_causal(name, [3100, i], c["lq"], c["lk"], c["hq"], c["hkv"], kv_dtype=c["kv"], q_dtype=c["q"],
                         page_size=c["page"], layout=c["layout"], kv_sigma=c["sigma"], q_sigma=c["q_sigma"],
                         softmax_scale=c["scale"], mode=c["mode"])


@pytest.mark.parametrize("i", range(N_CASES), ids=[f"{i}_{_draw(i)['mode']}" for i in range(N_CASES)])
def test_random_shape_parity(i):
    c = _draw(i)
    p = w.poison_unused(_problem(i, c))
    print(f"case {i}: {c}", flush=True)
    ref, ref_lse = oracle.attention(p)
    bits, lse = run_gpu(p, split=c.get("split"))
    out = bf16_bits_to_f64(bits)
    assert np.all(np.isfinite(out)), "non-finite output"
    # half a bf16 step at each reference value (7 stored mantissa bits)
    half_step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 8)
    beyond = float(np.max(np.abs(out - ref) - half_step))
    rl = refs.rel_l2(out, ref)
    print(f"random case {i}: error beyond bf16 rounding {beyond:.3e}, rel_l2 {rl:.3e} "
          f"(floor {refs.rel_l2(refs.bf16_round(ref), ref):.3e})", flush=True)
    assert beyond <= 1e-2, beyond
    assert rl <= 2e-3, rl
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), "lse finiteness differs"
    if fin.any():
        excess = np.abs(lse[fin] - ref_lse[fin]) - 5e-5 * np.abs(ref_lse[fin])
        assert float(np.max(excess)) <= 1e-3, float(np.max(excess))
