"""CPU checks of the benchmark's bookkeeping: the kernels it attributes times
and counters to exist in the HIP sources, the recorded profile data name
those kernels, and the kernel-trace summary picks out the cold calls."""
from __future__ import annotations

import json
import os
import re

import bench

CSRC = os.path.join(bench.ROOT, "paged_gqa_attention_hd256_amd", "csrc")


def _kernel_names():
    names = set()
    for f in os.listdir(CSRC):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f)) as fh:
                names.update(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+)\s*\(", fh.read()))
    return names


def test_benchmarked_kernels_exist():
    defined = _kernel_names()
    for mode, k in bench.KERNELS.items():
        assert k["main"] in defined, f"{mode}: {k['main']} is not a kernel in csrc/"
        for key in ("merge", "merge_tiles"):
            if key in k:
                assert k[key] in defined, f"{mode}: {k[key]} is not a kernel in csrc/"
        for f in k["sources"]:
            assert os.path.exists(os.path.join(CSRC, f)), f


def test_counter_records_name_the_benchmarked_kernel():
    with open(bench.COUNTERS) as fh:
        db = json.load(fh)
    for config, rec in db.items():
        k = bench.KERNELS[bench.mode_of(config)]
        assert rec["kernel"] == k["main"], f"{config}: counters of {rec['kernel']}, bench times {k['main']}"
        assert rec["hbm_bytes_per_launch"] > 0


def test_trace_summary_separates_cold_calls(tmp_path, capsys):
    """Cold calls are the library kernels that follow an eviction read; the
    settle, warmup and warm calls have none before them."""
    rows = [
        ("void pga::verify_kernel<2>(pga::VerifyArgs)", 0, 100),           # settle / warmup
        ("void pga::verify_merge_kernel<2>(pga::VerifyArgs)", 110, 120),
        ("at::native::reduce_kernel<512, 1>(...)", 200, 500),               # eviction read
        ("void pga::verify_kernel<2>(pga::VerifyArgs)", 510, 640),          # cold
        ("void pga::verify_merge_kernel<2>(pga::VerifyArgs)", 650, 670),    # cold
        ("void pga::verify_kernel<2>(pga::VerifyArgs)", 700, 800),          # warm
        ("void pga::(anonymous namespace)::quant_amax_kernel(pga::QuantArgs)", 900, 905),
    ]
    path = tmp_path / "trace.csv"
    with open(path, "w") as fh:
        fh.write("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for name, t0, t1 in rows:
            fh.write(f'KERNEL_DISPATCH,"{name}",{t0},{t1}\n')
    bench.trace_summary(str(path))
    out = json.loads(capsys.readouterr().out)
    v = out["pga::verify_kernel<2>"]
    assert v["dispatches"] == 3 and v["cold_calls"] == 1 and v["mean_us_cold"] == 0.13
    assert out["pga::verify_merge_kernel<2>"]["cold_calls"] == 1
    assert "pga::quant_amax_kernel" in out
