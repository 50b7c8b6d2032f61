"""Helpers for the GPU parity tests: run a problem through the HIP library and
compare with the fp64 oracle under the parity bar."""
from __future__ import annotations

import numpy as np

from tests import refs

MAX_ABS = 1e-2
REL_L2 = 2e-3
LSE_ABS = 1e-3


# Guard margins around every buffer the library writes: a write past either
# end of out, lse or the workspace lands in a margin and fails the test.
OUT_MARGIN = 4096          # bf16 elements (8 KiB) on each side of out
LSE_MARGIN = 1024          # fp32 elements on each side of lse
WS_MARGIN = 1 << 16        # bytes on each side of the workspace (keeps its 256-byte alignment)
OUT_SENTINEL = 0x7FA5      # a NaN pattern no kernel produces
LSE_SENTINEL = 0x7FC0DEAD    # another NaN pattern, compared as bits
WS_SENTINEL = 0xA5


class Guarded:
    """A device buffer with sentinel-filled margins on both sides; ``view`` is
    the part handed to the library."""

    def __init__(self, numel, dtype, margin, fill_bits, device="cuda"):
        import torch

        self.margin, self.numel = margin, numel
        bits_dtype = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.uint8: torch.uint8}[dtype]
        self.full = torch.empty(numel + 2 * margin, dtype=dtype, device=device)
        raw = self.full.view(bits_dtype)
        if bits_dtype == torch.int16 and fill_bits >= 1 << 15:
            fill_bits -= 1 << 16
        if bits_dtype == torch.int32 and fill_bits >= 1 << 31:
            fill_bits -= 1 << 32
        raw.fill_(fill_bits)
        self.bits_dtype = bits_dtype
        self.fill_bits = fill_bits
        self.view = self.full[margin:margin + numel]

    def check(self, what):
        raw = self.full.view(self.bits_dtype)
        head = raw[:self.margin].cpu()
        tail = raw[self.margin + self.numel:].cpu()
        bad_head = int((head != self.fill_bits).sum())
        bad_tail = int((tail != self.fill_bits).sum())
        assert bad_head == 0 and bad_tail == 0, \
            f"{what}: {bad_head} elements written before and {bad_tail} after the buffer"


def run_gpu(p, split=None, repeat=1, stage="all", with_lse=True, max_kv_len=None):
    """Run problem p through the library ``repeat`` times and return the output
    bits and lse of each run.  out, lse and the workspace sit inside sentinel
    margins that are checked after every run; with_lse=False passes no lse
    pointer (the returned lse is then all NaN); max_kv_len overrides the host
    bound of the key lengths."""
    import numpy as np
    import torch
    from paged_gqa_attention_hd256_amd import problem_io

    dp = problem_io.to_device(p, kv_split_tokens=split, max_kv_len=max_kv_len)
    g_out = Guarded(dp.out.numel(), torch.bfloat16, OUT_MARGIN, OUT_SENTINEL)
    dp.out = g_out.view.view(dp.out.shape)
    g_lse = None
    if with_lse:
        g_lse = Guarded(dp.lse.numel(), torch.float32, LSE_MARGIN, LSE_SENTINEL)
        dp.lse = g_lse.view.view(dp.lse.shape)
    else:
        dp.lse = None
    g_ws = None
    if dp.workspace is not None:
        g_ws = Guarded(dp.workspace.numel(), torch.uint8, WS_MARGIN, WS_SENTINEL)
        dp.workspace = g_ws.view
    outs = []
    for _ in range(repeat):
        dp.out.fill_(float("nan"))
        if dp.lse is not None:
            dp.lse.fill_(float("nan"))
        problem_io.run(dp, stage=stage)
        torch.cuda.synchronize()
        for g, what in ((g_out, "out"), (g_lse, "lse"), (g_ws, "workspace")):
            if g is not None:
                g.check(f"{p.name}: {what}")
        lse = dp.lse.cpu().numpy().copy() if dp.lse is not None else np.full(dp.out.shape[:2], np.nan, np.float32)
        outs.append((dp.out.view(torch.int16).cpu().numpy().copy(), lse))
    return outs if repeat > 1 else outs[0]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_parity(got_bits, got_lse, ref, ref_lse, rows=None, what="", check_lse=True):
    out = bf16_bits_to_f64(got_bits)
    if rows is not None:
        out, ref, got_lse, ref_lse = out[rows], ref[rows], got_lse[rows], ref_lse[rows]
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    ma, rl = refs.max_abs(out, ref), refs.rel_l2(out, ref)
    floor = refs.rel_l2(refs.bf16_round(ref), ref)
    print(f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e} (bf16 floor {floor:.3e})", flush=True)
    assert ma <= MAX_ABS, f"{what}: max_abs {ma}"
    assert rl <= REL_L2, f"{what}: rel_l2 {rl}"
    if not check_lse:
        return ma, rl
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin), f"{what}: lse finiteness differs"
    if fin.any():
        le = float(np.max(np.abs(got_lse[fin] - ref_lse[fin])))
        assert le <= LSE_ABS, f"{what}: lse abs err {le}"
    return ma, rl
