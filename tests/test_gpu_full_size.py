"""Full-size parity, in the launch configuration the benchmark times.

Every workload the benchmark measures is built at its full size and run once
through the C ABI the way the benchmark runs it (same problem, same split
setting, every stage of the call).  Sampled query rows, all heads of each, are
then checked against the fp64 oracle, which computes only those rows, under
the same bar as the small parity tests.  The verify workloads are checked row
for row in full; the others on the first and last row of every sequence
(the shortest and the longest context of a prefill) plus evenly spaced and
seeded random rows in between.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import workloads as w
from tests import gpu_util

pytestmark = pytest.mark.gpu

# The tiny verify workload is checked in full by test_gpu_parity.py.
FULL_SIZE = [n for n in w.config_names() if n != "tiny_verify"]
SAMPLED_ROWS = 192
THREADS = min(16, os.cpu_count() or 1)


def _sample(p, n: int = SAMPLED_ROWS) -> np.ndarray:
    if p.mode == "verify":
        return np.arange(p.num_tokens)
    cu = np.asarray(p.cu_seqlens_q, dtype=np.int64)
    rows = set()
    for b in range(p.num_seqs):
        if cu[b + 1] > cu[b]:
            rows.update((int(cu[b]), int(cu[b + 1]) - 1))
    rows.update(np.linspace(0, p.num_tokens - 1, n // 2).round().astype(np.int64).tolist())
    rng = np.random.default_rng(20261202)
    rows.update(rng.integers(0, p.num_tokens, size=n // 2).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_sampled_rows(name):
    p = w.config(name)
    rows = _sample(p)
    print(f"{name}: {p.num_tokens} query tokens x {p.num_q_heads} heads, checking {rows.size} rows", flush=True)
    got, got_lse = gpu_util.run_gpu(p)  # the problem's own split setting, as the benchmark uses
    ref_p = oracle.quantized_problem(p) if "k_new" in p.meta else p
    ref, ref_lse = oracle.attention(ref_p, rows=rows, threads=THREADS)
    gpu_util.assert_parity(got, got_lse, ref, ref_lse, rows=rows, what=f"{name} ({rows.size} rows)")
