"""Upload a host-side problem description to the GPU and run it.

``to_device`` accepts any object with the attributes of a paged-attention
problem (numpy arrays of raw bf16 / FP8 codes: ``q``, ``k_cache``,
``v_cache``, ``block_table``, ``cu_seqlens_q``, ``seq_lens_k``, optional
``indices``; scalars ``q_dtype``, ``kv_dtype``, descales, ``softmax_scale``,
``mode``, ``kv_layout``, ``kv_split_tokens``).  A prefill problem whose
``meta`` carries bf16 ``k_new`` / ``v_new`` (and ``q`` in bf16) runs as the
FP8 quantisation of Q and the new keys/values followed by the FP8 prefill.
It only moves data; the computation itself runs in the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import (PagedKV, paged_attn_prefill_prefix, paged_attn_verify, prefill_quantize_fp8, quantize_workspace_bytes,
               sparse_paged_attn, sparse_workspace_bytes, verify_workspace_bytes)


def _codes_to_tensor(codes: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(codes))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    else:
        t = t.view(torch.uint8).view(torch.float8_e4m3fn)
    return t.to(device)


def _scalar(x: float, device) -> torch.Tensor:
    return torch.tensor([x], dtype=torch.float32, device=device)


@dataclass
class QuantBuffers:
    """Inputs and outputs of the FP8 quantisation ahead of a prefill."""

    q_bf16: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    q_fp8: torch.Tensor
    q_descale: torch.Tensor
    workspace: torch.Tensor


@dataclass
class DeviceProblem:
    mode: str
    q: torch.Tensor
    q_descale: Optional[torch.Tensor]
    cu_seqlens_q: torch.Tensor
    seq_lens_k: torch.Tensor
    cu_seqlens_k: torch.Tensor
    kv: PagedKV
    softmax_scale: float
    max_q_len: int
    max_kv_len: int
    kv_split_tokens: int
    indices: Optional[torch.Tensor]
    out: torch.Tensor
    lse: torch.Tensor
    workspace: Optional[torch.Tensor]
    quant: Optional[QuantBuffers] = None


def to_device(p, device="cuda", kv_split_tokens: Optional[int] = None,
              max_kv_len: Optional[int] = None) -> DeviceProblem:
    """Device copies of problem p.  max_kv_len overrides the host bound of the
    key lengths (default: their maximum); the block table then gets columns
    of page 0 up to that bound, which no visible key reads."""
    q = _codes_to_tensor(p.q, p.q_dtype, device)
    k = _codes_to_tensor(p.k_cache, p.kv_dtype, device)
    v = _codes_to_tensor(p.v_cache, p.kv_dtype, device)
    bt_np = np.ascontiguousarray(p.block_table, dtype=np.int32)
    if max_kv_len is not None:
        cols = -(-int(max_kv_len) // int(p.page_size))
        if bt_np.shape[1] < cols:
            bt_np = np.pad(bt_np, ((0, 0), (0, cols - bt_np.shape[1])))
    bt = torch.from_numpy(np.ascontiguousarray(bt_np)).to(device)
    kv = PagedKV(k, v, bt, layout=p.kv_layout, k_descale=_scalar(p.k_descale, device),
                 v_descale=_scalar(p.v_descale, device))
    cu_q = torch.from_numpy(np.ascontiguousarray(p.cu_seqlens_q, dtype=np.int32)).to(device)
    lens_k = torch.from_numpy(np.ascontiguousarray(p.seq_lens_k, dtype=np.int32)).to(device)
    cu_k_np = np.zeros(len(p.seq_lens_k) + 1, dtype=np.int32)
    cu_k_np[1:] = np.cumsum(p.seq_lens_k)
    cu_k = torch.from_numpy(cu_k_np).to(device)
    idx = None
    if getattr(p, "indices", None) is not None:
        idx = torch.from_numpy(np.ascontiguousarray(p.indices, dtype=np.int32)).to(device)
    T, Hq = p.q.shape[0], p.q.shape[1]
    out = torch.empty((T, Hq, 256), dtype=torch.bfloat16, device=device)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=device)
    max_q = int(np.diff(p.cu_seqlens_q).max()) if len(p.seq_lens_k) else 0
    max_k = int(np.max(p.seq_lens_k)) if len(p.seq_lens_k) else 0
    if max_kv_len is not None:
        assert max_kv_len >= max_k, "max_kv_len below a key length"
        max_k = int(max_kv_len)
    split = p.kv_split_tokens if kv_split_tokens is None else kv_split_tokens
    ws = None
    if p.mode == "verify":
        need = verify_workspace_bytes(Hq, kv.num_kv_heads, len(p.seq_lens_k), max(1, max_q), max_k, split)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=device)
    if p.mode == "sparse" and idx is not None:
        need = sparse_workspace_bytes(Hq, kv.num_kv_heads, T, idx.shape[1])
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=device)
    q_ds = _scalar(p.q_descale, device) if p.q_dtype != "bf16" else None
    quant = None
    meta = getattr(p, "meta", None) or {}
    if p.mode == "prefill" and "k_new" in meta:
        quant = QuantBuffers(q, _codes_to_tensor(meta["k_new"], "bf16", device),
                             _codes_to_tensor(meta["v_new"], "bf16", device),
                             torch.empty(q.shape, dtype=torch.float8_e4m3fn, device=device),
                             torch.empty(1, dtype=torch.float32, device=device),
                             torch.empty(quantize_workspace_bytes(), dtype=torch.uint8, device=device))
    return DeviceProblem(p.mode, q, q_ds, cu_q, lens_k, cu_k, kv, float(p.softmax_scale), max_q, max_k, split, idx,
                         out, lse, ws, quant)


def quantize(dp: DeviceProblem, stream=None):
    """The FP8 quantisation of a quantising prefill problem: Q into
    ``dp.quant.q_fp8`` (dynamic descale into ``dp.quant.q_descale``), the new
    keys and values into the pool."""
    qb = dp.quant
    return prefill_quantize_fp8(qb.q_bf16, dp.kv, qb.k_new, qb.v_new, dp.cu_seqlens_q, dp.cu_seqlens_k,
                                q_fp8=qb.q_fp8, q_descale_out=qb.q_descale, workspace=qb.workspace, stream=stream)


def run(dp: DeviceProblem, stream=None, stage: str = "all") -> torch.Tensor:
    """One call of the entry point matching ``dp.mode``; writes dp.out / dp.lse.
    For verify, ``stage`` may select only the attention kernel or only the merge;
    for sparse, ``stage="unsplit"`` asks for the launch without list pieces."""
    if dp.mode == "verify":
        return paged_attn_verify(dp.q, dp.cu_seqlens_q, dp.seq_lens_k, dp.max_q_len, dp.max_kv_len, dp.kv,
                                 dp.softmax_scale, dp.kv_split_tokens, q_descale=dp.q_descale, workspace=dp.workspace,
                                 out=dp.out, lse=dp.lse, stream=stream, stage=stage)
    if dp.mode == "prefill" and dp.quant is not None:
        # stage "all": quantise, then attend; "quant" / "attn": one of the two
        if stage in ("all", "quant"):
            quantize(dp, stream)
        if stage == "quant":
            return dp.quant.q_fp8
        return paged_attn_prefill_prefix(dp.quant.q_fp8, dp.cu_seqlens_q, dp.cu_seqlens_k, dp.max_q_len,
                                         dp.max_kv_len, dp.kv, dp.softmax_scale, q_descale=dp.quant.q_descale,
                                         out=dp.out, lse=dp.lse, stream=stream)
    if dp.mode == "prefill":
        return paged_attn_prefill_prefix(dp.q, dp.cu_seqlens_q, dp.cu_seqlens_k, dp.max_q_len, dp.max_kv_len, dp.kv,
                                         dp.softmax_scale, q_descale=dp.q_descale, out=dp.out, lse=dp.lse,
                                         stream=stream)
    if dp.mode == "sparse":
        return sparse_paged_attn(dp.q, dp.cu_seqlens_q, dp.seq_lens_k, dp.indices, dp.kv, dp.softmax_scale,
                                 q_descale=dp.q_descale, workspace=dp.workspace, out=dp.out, lse=dp.lse, stream=stream,
                                 split=stage != "unsplit")
    raise ValueError(dp.mode)
