"""CPU checks of the benchmark's bookkeeping: the kernels it attributes times
and counters to exist in the HIP sources, and the recorded profile data name
those kernels."""
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
        if "merge" in k:
            assert k["merge"] in defined, f"{mode}: {k['merge']} is not a kernel in csrc/"
        for f in k["sources"]:
            assert os.path.exists(os.path.join(CSRC, f)), f


def test_counter_records_name_the_benchmarked_kernel():
    with open(bench.COUNTERS) as fh:
        db = json.load(fh)
    for config, rec in db.items():
        k = bench.KERNELS[bench.mode_of(config)]
        assert rec["kernel"] == k["main"], f"{config}: counters of {rec['kernel']}, bench times {k['main']}"
        assert rec["hbm_bytes_per_launch"] > 0
