"""Helpers for the GPU parity tests: run a problem through the HIP library and
compare with the fp64 oracle under the parity bar."""
from __future__ import annotations

import numpy as np

from tests import refs

MAX_ABS = 1e-2
REL_L2 = 2e-3
LSE_ABS = 1e-3


def run_gpu(p, split=None, repeat=1, stage="all"):
    import torch
    from paged_gqa_attention_hd256_amd import problem_io

    dp = problem_io.to_device(p, kv_split_tokens=split)
    outs = []
    for _ in range(repeat):
        dp.out.fill_(float("nan"))
        dp.lse.fill_(float("nan"))
        problem_io.run(dp, stage=stage)
        torch.cuda.synchronize()
        outs.append((dp.out.view(torch.int16).cpu().numpy().copy(), dp.lse.cpu().numpy().copy()))
    return outs if repeat > 1 else outs[0]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_parity(got_bits, got_lse, ref, ref_lse, rows=None, what=""):
    out = bf16_bits_to_f64(got_bits)
    if rows is not None:
        out, ref, got_lse, ref_lse = out[rows], ref[rows], got_lse[rows], ref_lse[rows]
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    ma, rl = refs.max_abs(out, ref), refs.rel_l2(out, ref)
    floor = refs.rel_l2(refs.bf16_round(ref), ref)
    print(f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e} (bf16 floor {floor:.3e})", flush=True)
    assert ma <= MAX_ABS, f"{what}: max_abs {ma}"
    assert rl <= REL_L2, f"{what}: rel_l2 {rl}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin), f"{what}: lse finiteness differs"
    if fin.any():
        le = float(np.max(np.abs(got_lse[fin] - ref_lse[fin])))
        assert le <= LSE_ABS, f"{what}: lse abs err {le}"
    return ma, rl
