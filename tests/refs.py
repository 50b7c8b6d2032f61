"""Test-side helpers: independent dense references and comparison metrics.

The dense reference gathers each sequence's keys with numpy fancy indexing
and hands the contiguous tensors to torch's fp64 scaled_dot_product_attention
with a boolean mask built by a library routine (``torch.tril``) or from the
index lists.  It shares nothing with the oracle beyond the inputs.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def decode_torch(codes: np.ndarray, dtype: str) -> torch.Tensor:
    """Codes -> float64 through torch's own dtype conversions."""
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if dtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16).to(torch.float64)
    return t.view(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)


def logical_kv(p, b: int):
    """K, V of sequence b as contiguous [Lk, Hkv, D] float64 (descales applied)."""
    lk = int(p.seq_lens_k[b])
    j = np.arange(lk)
    pages = p.block_table[b, j // p.page_size]
    slots = j % p.page_size
    if p.kv_layout == "NHD":
        k = p.k_cache[pages, slots]
        v = p.v_cache[pages, slots]
    else:
        k = p.k_cache[pages, :, slots]
        v = p.v_cache[pages, :, slots]
    return decode_torch(k, p.kv_dtype) * p.k_descale, decode_torch(v, p.kv_dtype) * p.v_descale


def dense_attention(p, mask_of=None):
    """fp64 reference via torch SDPA.  ``mask_of(b, lq, lk) -> bool [lq, lk]``;
    the default is the bottom-right causal mask from torch.tril."""
    q_all = decode_torch(p.q, p.q_dtype) * p.q_descale
    T, Hq, D = q_all.shape
    r = Hq // p.num_kv_heads
    out = torch.zeros((T, Hq, D), dtype=torch.float64)
    for b in range(p.num_seqs):
        s, e = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        lq, lk = e - s, int(p.seq_lens_k[b])
        if lq == 0:
            continue
        k, v = logical_kv(p, b)
        if mask_of is None:
            mask = torch.ones(lq, lk, dtype=torch.bool).tril(diagonal=lk - lq)
        else:
            mask = torch.as_tensor(mask_of(b, lq, lk), dtype=torch.bool)
        q = q_all[s:e].permute(1, 0, 2)                               # [Hq, lq, D]
        kk = k.permute(1, 0, 2).repeat_interleave(r, dim=0).contiguous()   # [Hq, lk, D]
        vv = v.permute(1, 0, 2).repeat_interleave(r, dim=0).contiguous()
        o = F.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, scale=p.softmax_scale)
        out[s:e] = o.permute(1, 0, 2)
    return out.numpy()


def sparse_mask_of(p):
    """Mask builder for sparse problems: row t sees exactly its valid entries."""
    def mask_of(b, lq, lk):
        s = int(p.cu_seqlens_q[b])
        m = np.zeros((lq, lk), dtype=bool)
        for t in range(lq):
            row = p.indices[s + t]
            row = row[(row >= 0) & (row < lk)]
            m[t, row] = True
        return m
    return mask_of


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def max_abs(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bf16, returned as float64 (via torch)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def repack(p, seed: int, layout: str = "NHD", extra_pages: int = 3, fill_code=None):
    """The same logical K/V placed in a different random page permutation and
    pool layout (pages not referenced are filled with ``fill_code``)."""
    import copy
    q = copy.copy(p)
    rng = np.random.Generator(np.random.PCG64(seed))
    P, H, D = p.page_size, p.num_kv_heads, p.head_dim
    need = [(int(l) + P - 1) // P for l in p.seq_lens_k]
    n_pages = sum(need) + extra_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    shape = (n_pages, P, H, D) if layout == "NHD" else (n_pages, H, P, D)
    dt = p.k_cache.dtype
    code = fill_code if fill_code is not None else 0
    k = np.full(shape, code, dtype=dt)
    v = np.full(shape, code, dtype=dt)
    table = np.full((p.num_seqs, max(need) + 2), -1, dtype=np.int32)
    off = 0
    for b in range(p.num_seqs):
        for i in range(need[b]):
            src = p.block_table[b, i]
            dst = perm[off]
            off += 1
            table[b, i] = dst
            ks, vs = p.k_cache[src], p.v_cache[src]
            if p.kv_layout != layout:
                ks, vs = np.swapaxes(ks, 0, 1), np.swapaxes(vs, 0, 1)
            k[dst], v[dst] = ks, vs
    q.k_cache, q.v_cache, q.block_table, q.kv_layout = k, v, table, layout
    return q
