"""Seeded synthetic workloads.

Every tensor is drawn from numpy PCG64 streams derived from one
``SeedSequence`` per workload, in the fixed order lengths -> Q -> K -> V ->
pool permutation -> sparse indices.  Large normal draws are split into fixed
chunks, each with its own child seed, so the result does not depend on how
many threads fill them.

Encodings produced here (bit patterns, stored as unsigned integers):

* bf16: round-to-nearest-even of the float32 draw (uint16 per element).
* OCP FP8 E4M3FN: a per-tensor descale ``amax / 448`` and the code
  ``RNE(x / descale)`` saturated to +-448 (uint8 per element).  The quantiser
  serves input synthesis only: every consumer reads the codes and the descale.

KV pool layout: ``[num_pages, page_size, num_kv_heads, 256]`` ("NHD", the
default) or ``[num_pages, num_kv_heads, page_size, 256]`` ("HND").  A
sequence's logical token j lives at page ``block_table[b][j // page_size]``,
slot ``j % page_size``.  Unused block-table entries hold -1.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEAD_DIM = 256
BF16 = "bf16"
FP8 = "fp8_e4m3"
# A NaN bit pattern per encoding, used to poison slots that must never be read.
NAN_CODE = {BF16: 0x7FC0, FP8: 0x7F}
_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(seed: np.random.SeedSequence, n: int, sigma: float = 1.0) -> np.ndarray:
    """float32 N(0, sigma^2) draws, chunked with per-chunk child seeds."""
    out = np.empty(n, dtype=np.float32)
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = seed.spawn(nch)

    def fill(i):
        g = np.random.Generator(np.random.PCG64(kids[i]))
        sl = out[i * _CHUNK:(i + 1) * _CHUNK]
        g.standard_normal(out=sl, dtype=np.float32)
        if sigma != 1.0:
            sl *= np.float32(sigma)

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (finite inputs)."""
    u = x.view(np.uint32)
    rnd = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rnd) >> 16).astype(np.uint16)


def _to_e4m3_codes(x: np.ndarray) -> tuple[np.ndarray, float]:
    """Per-tensor FP8 E4M3FN quantisation: (codes, descale)."""
    import torch

    amax = float(np.max(np.abs(x))) if x.size else 1.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    out = np.empty(x.shape, dtype=np.uint8)
    xf, of = x.reshape(-1), out.reshape(-1)
    nch = (xf.size + _CHUNK - 1) // _CHUNK

    def enc(i):
        sl = slice(i * _CHUNK, (i + 1) * _CHUNK)
        t = torch.from_numpy(xf[sl] / descale).clamp_(-448.0, 448.0)
        of[sl] = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    if nch <= 1:
        if xf.size:
            enc(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(enc, range(nch)))
    return out, float(descale)


def _encode(x: np.ndarray, dtype: str) -> tuple[np.ndarray, float]:
    if dtype == BF16:
        return _to_bf16_bits(x), 1.0
    if dtype == FP8:
        return _to_e4m3_codes(x)
    raise ValueError(dtype)


@dataclass
class Problem:
    """One attention call's inputs (host numpy arrays of raw codes)."""

    name: str
    mode: str                      # "verify" | "prefill" | "sparse"
    q: np.ndarray                  # [T, Hq, 256] codes
    q_dtype: str
    q_descale: float
    cu_seqlens_q: np.ndarray       # int32 [B+1]
    seq_lens_k: np.ndarray         # int32 [B]
    k_cache: np.ndarray            # pool codes, NHD or HND
    v_cache: np.ndarray
    kv_dtype: str
    k_descale: float
    v_descale: float
    block_table: np.ndarray        # int32 [B, W]
    page_size: int
    num_q_heads: int
    num_kv_heads: int
    softmax_scale: float
    kv_layout: str = "NHD"
    indices: Optional[np.ndarray] = None   # int32 [T, W] (sparse only)
    kv_split_tokens: int = 0               # verify: 0 = library's choice
    head_dim: int = HEAD_DIM
    meta: dict = field(default_factory=dict)

    # ---- derived sizes -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens_k.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q).astype(np.int64)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.seq_lens_k.max()) if self.num_seqs else 0

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def kv_elt_bytes(self) -> int:
        return 2 if self.kv_dtype == BF16 else 1

    def kv_strides(self) -> tuple[int, int, int]:
        """(page, token, head) element strides of the pool layout."""
        P, H, D = self.page_size, self.num_kv_heads, self.head_dim
        if self.kv_layout == "NHD":
            return (P * H * D, H * D, D)
        return (H * P * D, D, P * D)

    def token_seq(self) -> np.ndarray:
        """Sequence id of each query token."""
        return np.repeat(np.arange(self.num_seqs), self.q_lens)


def visible_pairs(p: Problem) -> int:
    """Number of visible (query token, key) pairs, per query head."""
    if p.mode == "sparse":
        seq = p.token_seq()
        lk = p.seq_lens_k[seq][:, None]
        ok = (p.indices >= 0) & (p.indices < lk)
        return int(ok.sum())
    tot = 0
    for b in range(p.num_seqs):
        lq, lk = int(p.q_lens[b]), int(p.seq_lens_k[b])
        # token t sees keys 0 .. lk - lq + t
        tot += lq * (lk - lq) + lq * (lq + 1) // 2
    return tot


def kv_bytes_read(p: Problem) -> int:
    """Algorithmic K+V bytes of a verify/prefill call: every key once."""
    return int(p.seq_lens_k.astype(np.int64).sum()) * p.num_kv_heads * p.head_dim * 2 * p.kv_elt_bytes


def gathered_bytes(p: Problem) -> int:
    """Sparse: K+V bytes gathered, one row per (selected entry, kv head)."""
    return visible_pairs(p) * p.num_kv_heads * p.head_dim * 2 * p.kv_elt_bytes


def _pool_and_table(rng, lens_k, page_size, pool_pages):
    pages_per_seq = [(int(l) + page_size - 1) // page_size for l in lens_k]
    need = sum(pages_per_seq)
    num_pages = max(need, pool_pages or 0)
    perm = rng.permutation(num_pages).astype(np.int32)
    width = max(1, max(pages_per_seq) if pages_per_seq else 1)
    table = np.full((len(lens_k), width), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[off:off + n]
        off += n
    return num_pages, table


def _draw_kv(ss_k, ss_v, num_pages, page_size, hkv, kv_dtype, sigma, layout):
    shape = (num_pages, page_size, hkv, HEAD_DIM) if layout == "NHD" else (num_pages, hkv, page_size, HEAD_DIM)
    n = int(np.prod(shape))
    kx = _normal(ss_k, n, sigma).reshape(shape)
    kc, kds = _encode(kx, kv_dtype)
    del kx
    vx = _normal(ss_v, n, sigma).reshape(shape)
    vc, vds = _encode(vx, kv_dtype)
    return kc, kds, vc, vds


def make_causal(name, seed, lens_q, lens_k, num_q_heads, num_kv_heads, *, kv_dtype=BF16, q_dtype=BF16,
                page_size=16, pool_pages=None, kv_sigma=1.0, q_sigma=1.0, layout="NHD", mode="verify",
                softmax_scale=1.0 / 16.0, kv_split_tokens=0) -> Problem:
    """Bottom-right causal problem (verify or prefill) with explicit lengths."""
    ss = np.random.SeedSequence(seed)
    s_len, s_q, s_k, s_v, s_perm, _ = ss.spawn(6)
    del s_len  # lengths are given explicitly here
    lens_q = np.asarray(lens_q, dtype=np.int32)
    lens_k = np.asarray(lens_k, dtype=np.int32)
    assert np.all(lens_k >= lens_q)
    T = int(lens_q.sum())
    qx = _normal(s_q, T * num_q_heads * HEAD_DIM, q_sigma).reshape(T, num_q_heads, HEAD_DIM)
    qc, qds = _encode(qx, q_dtype)
    del qx
    rng_perm = np.random.Generator(np.random.PCG64(s_perm))
    num_pages, table = _pool_and_table(rng_perm, lens_k, page_size, pool_pages)
    kc, kds, vc, vds = _draw_kv(s_k, s_v, num_pages, page_size, num_kv_heads, kv_dtype, kv_sigma, layout)
    cu = np.zeros(len(lens_q) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens_q)
    return Problem(name=name, mode=mode, q=qc, q_dtype=q_dtype, q_descale=qds, cu_seqlens_q=cu,
                   seq_lens_k=lens_k, k_cache=kc, v_cache=vc, kv_dtype=kv_dtype, k_descale=kds,
                   v_descale=vds, block_table=table, page_size=page_size, num_q_heads=num_q_heads,
                   num_kv_heads=num_kv_heads, softmax_scale=softmax_scale, kv_layout=layout,
                   kv_split_tokens=kv_split_tokens, meta={"seed": seed})


def make_sparse(name, seed, lens_q, lens_k, num_q_heads, num_kv_heads, num_selected, *, kv_dtype=BF16,
                page_size=16, pool_pages=None, kv_sigma=1.0, layout="NHD", softmax_scale=1.0 / 16.0,
                width=None, pad_fraction=0.0) -> Problem:
    """Sparse problem: row t of sequence b selects sorted unique logical positions
    drawn uniformly from its causal context [0, Lk - Lq + t].  Rows whose context
    is smaller than ``num_selected`` select all of it; the rest of the row is -1.
    ``pad_fraction`` additionally blanks a random share of entries to -1."""
    ss = np.random.SeedSequence(seed)
    _, s_q, s_k, s_v, s_perm, s_idx = ss.spawn(6)
    lens_q = np.asarray(lens_q, dtype=np.int32)
    lens_k = np.asarray(lens_k, dtype=np.int32)
    T = int(lens_q.sum())
    qx = _normal(s_q, T * num_q_heads * HEAD_DIM).reshape(T, num_q_heads, HEAD_DIM)
    qc, _ = _encode(qx, BF16)
    del qx
    rng_perm = np.random.Generator(np.random.PCG64(s_perm))
    num_pages, table = _pool_and_table(rng_perm, lens_k, page_size, pool_pages)
    kc, kds, vc, vds = _draw_kv(s_k, s_v, num_pages, page_size, num_kv_heads, kv_dtype, kv_sigma, layout)
    W = width if width is not None else num_selected
    idx = np.full((T, W), -1, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(s_idx))
    row = 0
    for b in range(len(lens_q)):
        lq, lk = int(lens_q[b]), int(lens_k[b])
        for t in range(lq):
            ctx = lk - lq + t + 1
            n = min(num_selected, ctx, W)
            sel = np.sort(rng.choice(ctx, n, replace=False)).astype(np.int32)
            idx[row, :n] = sel
            row += 1
    if pad_fraction > 0:
        blank = rng.random(idx.shape) < pad_fraction
        idx[blank] = -1
    cu = np.zeros(len(lens_q) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens_q)
    return Problem(name=name, mode="sparse", q=qc, q_dtype=BF16, q_descale=1.0, cu_seqlens_q=cu,
                   seq_lens_k=lens_k, k_cache=kc, v_cache=vc, kv_dtype=kv_dtype, k_descale=kds,
                   v_descale=vds, block_table=table, page_size=page_size, num_q_heads=num_q_heads,
                   num_kv_heads=num_kv_heads, softmax_scale=softmax_scale, kv_layout=layout,
                   indices=idx, meta={"seed": seed})


def make_prefill_quant(name, seed, lens_q, lens_k, num_q_heads, num_kv_heads, *, page_size=16, layout="NHD",
                       q_sigma=1.0, kv_sigma=1.0, pool_pages=None) -> Problem:
    """Prefix-hit prefill inputs as they stand before the casts to FP8.

    The cached prefix sits in an FP8 pool under static per-tensor descales; Q
    and the new tokens' keys and values are bf16: ``p.q`` holds Q's bf16
    patterns, ``meta['k_new']`` / ``meta['v_new']`` the new keys and values
    ``[T, Hkv, 256]`` (token order of cu_seqlens_q) and ``meta['cu_seqlens_k']``
    the cumulative key lengths.  The pool slots of the new positions hold NaN
    codes until something writes them.
    """
    p = make_causal(name, seed, lens_q, lens_k, num_q_heads, num_kv_heads, kv_dtype=FP8, q_dtype=BF16,
                    page_size=page_size, pool_pages=pool_pages, kv_sigma=kv_sigma, q_sigma=q_sigma,
                    layout=layout, mode="prefill")
    s_kn, s_vn = np.random.SeedSequence(list(np.atleast_1d(seed)) + [7]).spawn(2)
    T = p.num_tokens
    n = T * num_kv_heads * HEAD_DIM
    p.meta["k_new"] = _to_bf16_bits(_normal(s_kn, n, kv_sigma)).reshape(T, num_kv_heads, HEAD_DIM)
    p.meta["v_new"] = _to_bf16_bits(_normal(s_vn, n, kv_sigma)).reshape(T, num_kv_heads, HEAD_DIM)
    cu_k = np.zeros(p.num_seqs + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(p.seq_lens_k)
    p.meta["cu_seqlens_k"] = cu_k
    nan = NAN_CODE[FP8]
    for b in range(p.num_seqs):
        lq = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        lk = int(p.seq_lens_k[b])
        pos = np.arange(lk - lq, lk)
        pages, slots = p.block_table[b, pos // page_size], pos % page_size
        if layout == "NHD":
            p.k_cache[pages, slots] = nan
            p.v_cache[pages, slots] = nan
        else:
            p.k_cache[pages, :, slots] = nan
            p.v_cache[pages, :, slots] = nan
    return p


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------
_CONFIGS = {
    "tiny_verify": 1,
    "mtp_verify_fp8": 2,
    "mtp_verify_gqa32": 3,
    "prefix_prefill_32k": 4,
    "prefix_prefill_128k": 4,
    "sparse_bf16": 5,
    "sparse_fp8": 5,
    "sparse_fp8_260rows": 6,
    "prefill_quant_32k": 7,
    # The shapes beyond the five named workloads: q_len 1, other GQA ratios,
    # bf16 prefill, a 64-token page in the head-major layout.
    "verify_decode_fp8": 8,
    "mtp_verify_fp8_6to1": 9,
    "sparse_fp8_3to1": 10,
    "prefix_prefill_32k_bf16": 11,
    "prefix_prefill_32k_page64_hnd": 12,
    "prefix_prefill_32k_bf16q": 13,
}


def config_names():
    return list(_CONFIGS)


def config(name: str) -> Problem:
    """Build one of the named full-size workloads (seed = its config index)."""
    c = _CONFIGS[name]
    if name == "tiny_verify":
        # B=2, q_len 2, 16 q / 1 kv, KV 600 and 1000 tokens, BF16, 128-page pool.
        return make_causal(name, [c, 0], [2, 2], [600, 1000], 16, 1, kv_dtype=BF16, q_dtype=BF16,
                           pool_pages=128, mode="verify")
    if name == "mtp_verify_fp8":
        # B=64, q_len 4, 16 q / 1 kv, KV lengths uniform in [2048, 32768], FP8 KV (sigma 0.5).
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c, 0]).spawn(6)[0]))
        lens_k = rng.integers(2048, 32768, size=64, endpoint=True)
        return make_causal(name, [c, 0], [4] * 64, lens_k, 16, 1, kv_dtype=FP8, q_dtype=BF16,
                           kv_sigma=0.5, mode="verify")
    if name == "mtp_verify_gqa32":
        # B=128, q_len 3, 32 q / 2 kv, KV lengths log-uniform in [513, 65536], FP8 KV,
        # split-KV segments of 4096 tokens.
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c, 0]).spawn(6)[0]))
        u = rng.uniform(math.log(513), math.log(65536), size=128)
        lens_k = np.clip(np.rint(np.exp(u)), 513, 65536).astype(np.int64)
        return make_causal(name, [c, 0], [3] * 128, lens_k, 32, 2, kv_dtype=FP8, q_dtype=BF16,
                           kv_sigma=0.5, mode="verify", kv_split_tokens=4096)
    if name in ("prefix_prefill_32k", "prefix_prefill_128k"):
        # 1 sequence, 8 q / 1 kv, 16384 new tokens after a 16384 / 114688-token cached prefix.
        lk = 32768 if name.endswith("32k") else 131072
        sub = 0 if name.endswith("32k") else 1
        return make_causal(name, [c, sub], [16384], [lk], 8, 1, kv_dtype=FP8, q_dtype=FP8,
                           mode="prefill")
    if name == "prefill_quant_32k":
        # The 16k-new / 32k-context prefill before its casts to FP8: bf16 Q and
        # new K/V, the 16384-token prefix already in the FP8 pool.
        return make_prefill_quant(name, [c, 0], [16384], [32768], 8, 1)
    if name == "sparse_fp8_260rows":
        # The few-row regime of the same selection: the last 260 rows of the
        # 32768-token sequence, 24 q / 2 kv, 2051 selected tokens each, FP8 K/V.
        return make_sparse(name, [c, 0], [260], [32768], 24, 2, 2051, kv_dtype=FP8)
    if name in ("verify_decode_fp8", "mtp_verify_fp8_6to1"):
        # The FP8 verify batch (64 sequences, KV lengths uniform in [2048, 32768])
        # as plain decode (q_len 1, 16 q / 1 kv) and at 6 q / 1 kv (q_len 4).
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c, 0]).spawn(6)[0]))
        lens_k = rng.integers(2048, 32768, size=64, endpoint=True)
        lq, hq = (1, 16) if name == "verify_decode_fp8" else (4, 6)
        return make_causal(name, [c, 0], [lq] * 64, lens_k, hq, 1, kv_dtype=FP8, q_dtype=BF16,
                           kv_sigma=0.5, mode="verify")
    if name == "sparse_fp8_3to1":
        # The sparse selection at 3 q / 1 kv (24 q / 8 kv heads split eight ways):
        # 8192 rows at positions 24576..32767, 2051 selected tokens each, FP8 K/V.
        return make_sparse(name, [c, 0], [8192], [32768], 3, 1, 2051, kv_dtype=FP8)
    if name == "prefix_prefill_32k_bf16":
        # The 16k-new / 32k-context prefill in bf16 (Q, K and V).
        return make_causal(name, [c, 0], [16384], [32768], 8, 1, kv_dtype=BF16, q_dtype=BF16, mode="prefill")
    if name == "prefix_prefill_32k_bf16q":
        # The 16k-new / 32k-context prefill with bf16 queries against the FP8 pool.
        return make_causal(name, [c, 0], [16384], [32768], 8, 1, kv_dtype=FP8, q_dtype=BF16, mode="prefill")
    if name == "prefix_prefill_32k_page64_hnd":
        # The FP8 16k / 32k prefill over 64-token pages laid out [pages, heads, slots, d].
        return make_causal(name, [c, 0], [16384], [32768], 8, 1, kv_dtype=FP8, q_dtype=FP8, page_size=64,
                           layout="HND", mode="prefill")
    if name in ("sparse_bf16", "sparse_fp8"):
        # 8192 query rows at positions 24576..32767 of one 32768-token sequence, 24 q / 2 kv,
        # 2051 selected tokens per row; the same draws encoded as BF16 or FP8 K/V.
        kvd = BF16 if name == "sparse_bf16" else FP8
        return make_sparse(name, [c, 0], [8192], [32768], 24, 2, 2051, kv_dtype=kvd)
    raise KeyError(name)


def poison_unused(p: Problem) -> Problem:
    """Write NaN codes into every pool slot that no visible key maps to.

    For causal problems that is every slot at or past each sequence's KV length
    and every page the block table does not reference; for sparse problems only
    the selected entries stay finite, so a read of any other slot shows up as NaN.
    """
    nan = NAN_CODE[p.kv_dtype]
    P = p.page_size
    keep = np.zeros((p.num_pages, P), dtype=bool)  # (page, slot) holds a visible key
    seq_of_row = p.token_seq()
    for b in range(p.num_seqs):
        lk = int(p.seq_lens_k[b])
        if p.mode == "sparse":
            rows = np.nonzero(seq_of_row == b)[0]
            sel = p.indices[rows].reshape(-1)
            sel = np.unique(sel[(sel >= 0) & (sel < lk)])
        else:
            sel = np.arange(lk)
        pages = p.block_table[b, sel // P]
        keep[pages, sel % P] = True
    k = p.k_cache
    v = p.v_cache
    if p.kv_layout == "NHD":
        k[~keep] = nan
        v[~keep] = nan
    else:
        mask = np.broadcast_to(~keep[:, None, :], k.shape[:3])
        k[mask] = nan
        v[mask] = nan
    p.meta["poisoned"] = True
    return p


def sample_rows(p: Problem, n: int, seed: int = 0) -> np.ndarray:
    """A deterministic sample of query-token indices for sampled parity at full
    size: the first and last token of every sequence (capped) plus uniform draws."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    cu = p.cu_seqlens_q
    edge = set()
    for b in range(p.num_seqs):
        if cu[b + 1] > cu[b]:
            edge.add(int(cu[b]))
            edge.add(int(cu[b + 1]) - 1)
    edge = sorted(edge)
    if len(edge) > n // 2:
        pick = rng.choice(len(edge), n // 2, replace=False)
        edge = sorted(edge[i] for i in pick)
    rest = n - len(edge)
    extra = rng.choice(p.num_tokens, min(rest, p.num_tokens), replace=False) if rest > 0 else []
    return np.unique(np.concatenate([np.asarray(edge, dtype=np.int64), np.asarray(extra, dtype=np.int64)]))
