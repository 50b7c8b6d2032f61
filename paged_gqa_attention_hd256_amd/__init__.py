"""Paged grouped-query attention, head_dim 256, for MI355X (gfx950).

A thin ctypes binding over ``libpaged_gqa.so`` (the C ABI in
``include/paged_gqa.h``).  The functions here only marshal torch tensors into
pointers, sizes and the current HIP stream; every step of the computation runs
in the library's HIP kernels.  PyTorch provides device memory and streams.

If the library has not been built, importing works but every call raises
``LibraryNotBuilt``: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "PagedKV", "paged_attn_verify", "paged_attn_verify_noalloc", "paged_attn_prefill_prefix", "sparse_paged_attn",
    "sparse_splits", "sparse_gather_sum", "verify_gather_sum", "sparse_workspace_bytes", "prefill_quantize_fp8", "quantize_workspace_bytes", "validate_inputs",
    "verify_workspace_bytes", "verify_split_tokens", "status_string", "abi_version", "library_path",
    "PagedGQAError", "LibraryNotBuilt", "load_library",
]

HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(HERE, "libpaged_gqa.so")

BF16, FP8 = 1, 2
OK = 0


class PagedGQAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {status_string(status)}")
        self.status = status


class LibraryNotBuilt(RuntimeError):
    pass


class _KV(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("k_stride_page", ctypes.c_int64), ("k_stride_token", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_page", ctypes.c_int64), ("v_stride_token", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
        ("k_descale", ctypes.c_void_p), ("v_descale", ctypes.c_void_p),
    ]


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _SO


def load_library():
    """Load libpaged_gqa.so (raises LibraryNotBuilt if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                raise LibraryNotBuilt(f"{_SO} is missing: build it with paged_gqa_attention_hd256_amd.build.build()")
            lib = ctypes.CDLL(_SO)
            P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
            KVP = ctypes.POINTER(_KV)
            for fn in ("paged_attn_verify", "paged_attn_verify_partials", "paged_attn_verify_merge"):
                getattr(lib, fn).argtypes = [P, I32, P, I32, I32, P, P, I32, I32, KVP, F, I32, P, SZ, P, P, P]
                getattr(lib, fn).restype = ctypes.c_int
            lib.paged_attn_verify_noalloc.argtypes = [P, I32, P, I32, I32, P, P, I32, I32, KVP, F, I32, P, P, P]
            lib.paged_attn_verify_noalloc.restype = ctypes.c_int
            lib.paged_attn_verify_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
            lib.paged_attn_verify_workspace_bytes.restype = SZ
            lib.paged_attn_verify_split_tokens.argtypes = [I32, I32, I32, I32, I32, I32]
            lib.paged_attn_verify_split_tokens.restype = I32
            lib.paged_attn_prefill_prefix.argtypes = [P, I32, P, I32, I32, P, P, I32, I32, KVP, F, P, P, P]
            lib.paged_attn_prefill_prefix.restype = ctypes.c_int
            lib.sparse_paged_attn.argtypes = [P, I32, P, I32, I32, I32, P, P, P, I64, I32, KVP, F, P, SZ, P, P, P]
            lib.sparse_paged_attn.restype = ctypes.c_int
            lib.sparse_gather_sum.argtypes = [I32, I32, P, P, P, I64, I32, KVP, P, P]
            lib.sparse_gather_sum.restype = ctypes.c_int
            lib.paged_attn_verify_gather_sum.argtypes = [I32, P, P, I32, I32, KVP, I32, P, P]
            lib.paged_attn_verify_gather_sum.restype = ctypes.c_int
            lib.sparse_paged_attn_splits.argtypes = [I32, I32, I32, I32]
            lib.sparse_paged_attn_splits.restype = I32
            lib.sparse_paged_attn_workspace_bytes.argtypes = [I32, I32, I32, I32]
            lib.sparse_paged_attn_workspace_bytes.restype = SZ
            lib.prefill_quantize_fp8.argtypes = [P, I32, I32, P, P, P, P, P, I32, P, P, ctypes.c_void_p, P, SZ, P]
            lib.prefill_quantize_fp8.restype = ctypes.c_int
            lib.prefill_quantize_fp8_workspace_bytes.argtypes = []
            lib.prefill_quantize_fp8_workspace_bytes.restype = SZ
            lib.pga_validate_inputs.argtypes = [I32, I32, P, P, P, I32, I32, KVP, P, I64, I32, P, P, P]
            lib.pga_validate_inputs.restype = ctypes.c_int
            lib.pga_status_string.argtypes = [ctypes.c_int]
            lib.pga_status_string.restype = ctypes.c_char_p
            lib.pga_abi_version.argtypes = []
            lib.pga_abi_version.restype = ctypes.c_int
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().pga_status_string(status).decode()


def abi_version() -> int:
    return load_library().pga_abi_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8
    raise TypeError(f"unsupported dtype {t.dtype}: expected bfloat16 or float8_e4m3fn")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclass
class PagedKV:
    """A paged KV pool.  ``k_cache``/``v_cache`` are 4-D with the head dimension
    last: ``[pages, page_size, kv_heads, 256]`` (layout "NHD") or
    ``[pages, kv_heads, page_size, 256]`` ("HND"); any strides are passed on.
    ``block_table`` is int32 ``[num_seqs, width]``; descales are 1-element fp32
    device tensors or None."""

    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    layout: str = "NHD"
    k_descale: Optional[torch.Tensor] = None
    v_descale: Optional[torch.Tensor] = None

    def _struct(self) -> _KV:
        k, v = self.k_cache, self.v_cache
        if k.dim() != 4 or v.dim() != 4:
            raise ValueError("k_cache and v_cache must be 4-D")
        if self.layout == "NHD":
            page_size, heads = k.shape[1], k.shape[2]
            ks, vs = (k.stride(0), k.stride(1), k.stride(2)), (v.stride(0), v.stride(1), v.stride(2))
        elif self.layout == "HND":
            page_size, heads = k.shape[2], k.shape[1]
            ks, vs = (k.stride(0), k.stride(2), k.stride(1)), (v.stride(0), v.stride(2), v.stride(1))
        else:
            raise ValueError(self.layout)
        if k.stride(3) != 1 or v.stride(3) != 1:
            raise ValueError("the head dimension must be unit-stride")
        if self.block_table.dtype != torch.int32:
            raise TypeError("block_table must be int32")
        s = _KV()
        s.k_cache, s.v_cache = k.data_ptr(), v.data_ptr()
        s.dtype = _dtype_code(k)
        s.num_kv_heads, s.head_dim, s.page_size = heads, k.shape[3], page_size
        s.num_pages, s.reserved = k.shape[0], 0
        s.k_stride_page, s.k_stride_token, s.k_stride_head = ks
        s.v_stride_page, s.v_stride_token, s.v_stride_head = vs
        s.block_table = self.block_table.data_ptr()
        s.block_table_stride = self.block_table.stride(0) if self.block_table.dim() == 2 else 0
        s.k_descale, s.v_descale = _ptr(self.k_descale), _ptr(self.v_descale)
        return s

    @property
    def num_kv_heads(self) -> int:
        return self.k_cache.shape[2] if self.layout == "NHD" else self.k_cache.shape[1]


def _check(fn: str, status: int):
    if status != OK:
        raise PagedGQAError(fn, status)


def verify_workspace_bytes(num_q_heads, num_kv_heads, num_seqs, max_q_len, max_kv_len, kv_split_tokens=0) -> int:
    return load_library().paged_attn_verify_workspace_bytes(num_q_heads, num_kv_heads, num_seqs, max_q_len,
                                                            max_kv_len, kv_split_tokens)


def verify_split_tokens(num_q_heads, num_kv_heads, num_seqs, max_q_len, max_kv_len, kv_split_tokens=0) -> int:
    return load_library().paged_attn_verify_split_tokens(num_q_heads, num_kv_heads, num_seqs, max_q_len,
                                                         max_kv_len, kv_split_tokens)


def _out(q: torch.Tensor, out):
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    return out


_VERIFY_STAGE = {"all": "paged_attn_verify", "partials": "paged_attn_verify_partials",
                 "merge": "paged_attn_verify_merge"}


def paged_attn_verify(q, cu_seqlens_q, seq_lens_k, max_q_len: int, max_kv_len: int, kv: PagedKV,
                      softmax_scale: float, kv_split_tokens: int = 0, q_descale=None, workspace=None,
                      out=None, lse=None, stream=None, stage: str = "all"):
    """Speculative-verify attention; returns ``out`` ([T, Hq, 256] bf16).
    ``stage`` selects both kernels ("all"), only the attention kernel
    ("partials") or only the log-sum-exp merge ("merge")."""
    lib = load_library()
    fn = _VERIFY_STAGE[stage]
    hq = q.shape[1]
    need = verify_workspace_bytes(hq, kv.num_kv_heads, seq_lens_k.shape[0], max_q_len, max_kv_len, kv_split_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = _out(q, out)
    s = kv._struct()
    st = getattr(lib, fn)(q.data_ptr(), _dtype_code(q), _ptr(q_descale), hq, seq_lens_k.shape[0],
                               cu_seqlens_q.data_ptr(), seq_lens_k.data_ptr(), max_q_len, max_kv_len,
                               ctypes.byref(s), float(softmax_scale), kv_split_tokens, _ptr(workspace),
                               0 if workspace is None else workspace.numel() * workspace.element_size(),
                               out.data_ptr(), _ptr(lse), _stream(stream))
    _check(fn, st)
    return out


def paged_attn_verify_noalloc(q, cu_seqlens_q, seq_lens_k, max_q_len: int, max_kv_len: int, kv: PagedKV,
                              softmax_scale: float, out, kv_split_tokens: int = 0, q_descale=None, lse=None,
                              stream=None):
    """paged_attn_verify without a workspace: the library keeps the partials in
    its fixed per-device scratch (PGA_VERIFY_NOALLOC_SCRATCH_BYTES) and
    allocates nothing.  ``out`` must be given (this wrapper allocates nothing
    either).  Calls that may overlap on one device must be serialised."""
    lib = load_library()
    s = kv._struct()
    st = lib.paged_attn_verify_noalloc(q.data_ptr(), _dtype_code(q), _ptr(q_descale), q.shape[1],
                                       seq_lens_k.shape[0], cu_seqlens_q.data_ptr(), seq_lens_k.data_ptr(),
                                       max_q_len, max_kv_len, ctypes.byref(s), float(softmax_scale), kv_split_tokens,
                                       out.data_ptr(), _ptr(lse), _stream(stream))
    _check("paged_attn_verify_noalloc", st)
    return out


def paged_attn_prefill_prefix(q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, kv: PagedKV,
                              softmax_scale: float, q_descale=None, out=None, lse=None, stream=None):
    """Prefill against a cached prefix (bottom-right causal); returns ``out``."""
    lib = load_library()
    out = _out(q, out)
    s = kv._struct()
    st = lib.paged_attn_prefill_prefix(q.data_ptr(), _dtype_code(q), _ptr(q_descale), q.shape[1],
                                       cu_seqlens_q.shape[0] - 1, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                                       max_seqlen_q, max_seqlen_k, ctypes.byref(s), float(softmax_scale),
                                       out.data_ptr(), _ptr(lse), _stream(stream))
    _check("paged_attn_prefill_prefix", st)
    return out


def sparse_splits(num_q_heads: int, num_kv_heads: int, num_q_tokens: int, num_selected: int) -> int:
    return load_library().sparse_paged_attn_splits(num_q_heads, num_kv_heads, num_q_tokens, num_selected)


def sparse_workspace_bytes(num_q_heads: int, num_kv_heads: int, num_q_tokens: int, num_selected: int) -> int:
    return load_library().sparse_paged_attn_workspace_bytes(num_q_heads, num_kv_heads, num_q_tokens, num_selected)


def sparse_paged_attn(q, cu_seqlens_q, seq_lens_k, indices, kv: PagedKV, softmax_scale: float,
                      num_selected: Optional[int] = None, q_descale=None, workspace=None, out=None, lse=None,
                      stream=None, split: bool = True):
    """Selected-token attention; ``indices`` is int32 [T, W]; returns ``out``.
    With ``split`` (the default) the library may cut each row's list into
    pieces when there are few rows; ``workspace`` is then allocated here
    unless given.  ``split=False`` asks for the unsplit launch."""
    lib = load_library()
    out = _out(q, out)
    s = kv._struct()
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.stride(1) != 1:
        raise ValueError("indices must be a row-major int32 [T, W] tensor")
    ns = indices.shape[1] if num_selected is None else num_selected
    if not split:
        workspace = None
    elif workspace is None:
        need = sparse_workspace_bytes(q.shape[1], kv.num_kv_heads, q.shape[0], ns)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib.sparse_paged_attn(q.data_ptr(), _dtype_code(q), _ptr(q_descale), q.shape[1], q.shape[0],
                               seq_lens_k.shape[0], cu_seqlens_q.data_ptr(), seq_lens_k.data_ptr(),
                               indices.data_ptr(), indices.stride(0), ns, ctypes.byref(s), float(softmax_scale),
                               _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                               out.data_ptr(), _ptr(lse), _stream(stream))
    _check("sparse_paged_attn", st)
    return out


def sparse_gather_sum(cu_seqlens_q, seq_lens_k, indices, kv: PagedKV, num_selected: Optional[int] = None,
                      out=None, stream=None):
    """Measurement helper: the same-index gather of ``sparse_paged_attn``
    (the K and V rows each row's valid entries select, per kv head), summed
    as 32-bit words; returns uint32-valued int32 ``out`` [T, Hkv, row words]."""
    lib = load_library()
    s = kv._struct()
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.stride(1) != 1:
        raise ValueError("indices must be a row-major int32 [T, W] tensor")
    ns = indices.shape[1] if num_selected is None else num_selected
    words = 256 * (1 if s.dtype == FP8 else 2) // 4
    if out is None:
        out = torch.empty((indices.shape[0], kv.num_kv_heads, words), dtype=torch.int32, device=indices.device)
    st = lib.sparse_gather_sum(indices.shape[0], seq_lens_k.shape[0], cu_seqlens_q.data_ptr(), seq_lens_k.data_ptr(),
                               indices.data_ptr(), indices.stride(0), ns, ctypes.byref(s), out.data_ptr(),
                               _stream(stream))
    _check("sparse_gather_sum", st)
    return out


def verify_gather_sum(cu_seqlens_q, seq_lens_k, max_q_len: int, max_kv_len: int, kv: PagedKV,
                      kv_split_tokens: int = 0, out=None, stream=None):
    """Measurement helper: the page gather of ``paged_attn_verify`` on its own
    work split (the K and V rows of every key below each history's length, per
    kv head), summed as 32-bit words and added into uint32-valued int32
    ``out`` [num_seqs, Hkv] (zeros when not given), which it returns."""
    lib = load_library()
    s = kv._struct()
    if out is None:
        out = torch.zeros((seq_lens_k.shape[0], kv.num_kv_heads), dtype=torch.int32, device=seq_lens_k.device)
    st = lib.paged_attn_verify_gather_sum(seq_lens_k.shape[0], cu_seqlens_q.data_ptr(), seq_lens_k.data_ptr(),
                                          int(max_q_len), int(max_kv_len), ctypes.byref(s), int(kv_split_tokens or 0),
                                          out.data_ptr(), _stream(stream))
    _check("paged_attn_verify_gather_sum", st)
    return out


def quantize_workspace_bytes() -> int:
    return load_library().prefill_quantize_fp8_workspace_bytes()


def prefill_quantize_fp8(q, kv: Optional[PagedKV] = None, k_new=None, v_new=None, cu_seqlens_q=None,
                         cu_seqlens_k=None, q_descale=None, q_fp8=None, q_descale_out=None, workspace=None,
                         stream=None):
    """Per-tensor FP8 quantisation ahead of the FP8 prefill.  Codes bf16 ``q``
    ([T, Hq, 256]) into ``q_fp8`` (float8_e4m3fn) with the descale ``q_descale``
    (a 1-element fp32 tensor) or, when that is None, the dynamic descale
    amax/448, which lands in ``q_descale_out``; with ``k_new``/``v_new``
    ([T, Hkv, 256] bf16) it also writes the new tokens' keys and values into
    ``kv``'s FP8 pool under the pool's descales.  Returns (q_fp8, q_descale_out)."""
    lib = load_library()
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [T, Hq, 256] tensor")
    if q_fp8 is None:
        q_fp8 = torch.empty(q.shape, dtype=torch.float8_e4m3fn, device=q.device)
    if q_descale_out is None:
        q_descale_out = torch.empty(1, dtype=torch.float32, device=q.device)
    if q_descale is None and workspace is None:
        workspace = torch.empty(quantize_workspace_bytes(), dtype=torch.uint8, device=q.device)
    s = kv._struct() if kv is not None else None
    for t in (k_new, v_new):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous()):
            raise ValueError("k_new / v_new must be contiguous bf16 [T, Hkv, 256] tensors")
    num_seqs = cu_seqlens_q.shape[0] - 1 if cu_seqlens_q is not None else 0
    st = lib.prefill_quantize_fp8(q.data_ptr(), q.shape[1], q.shape[0], _ptr(q_descale), q_fp8.data_ptr(),
                                  q_descale_out.data_ptr(), _ptr(k_new), _ptr(v_new), num_seqs, _ptr(cu_seqlens_q),
                                  _ptr(cu_seqlens_k), None if s is None else ctypes.addressof(s), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  _stream(stream))
    _check("prefill_quantize_fp8", st)
    return q_fp8, q_descale_out


def validate_inputs(cu_seqlens_q, kv: PagedKV, seq_lens_k=None, cu_seqlens_k=None, max_q_len: int = 0,
                    max_kv_len: int = 0, indices=None, num_selected: Optional[int] = None, stream=None):
    """Check the device data the attention calls take on trust (lengths, block
    table, index lists); synchronous.  Returns (status, counts) with counts =
    [invalid-length sequences, sequences beyond the bounds, bad block-table
    entries, index entries past Lk]; status is 0 or PGA_ERR_INVALID_DATA (7)."""
    lib = load_library()
    s = kv._struct()
    counts = torch.empty(4, dtype=torch.int32, device=cu_seqlens_q.device)
    host = (ctypes.c_int32 * 4)()
    num_seqs = cu_seqlens_q.shape[0] - 1
    ntok = -1
    stride, ns = 0, 0
    if indices is not None:
        if indices.dtype != torch.int32 or indices.dim() != 2 or indices.stride(1) != 1:
            raise ValueError("indices must be a row-major int32 [T, W] tensor")
        ntok, stride = indices.shape[0], indices.stride(0)
        ns = indices.shape[1] if num_selected is None else num_selected
    st = lib.pga_validate_inputs(num_seqs, ntok, cu_seqlens_q.data_ptr(), _ptr(seq_lens_k), _ptr(cu_seqlens_k),
                                 max_q_len, max_kv_len, ctypes.byref(s), _ptr(indices), stride, ns,
                                 counts.data_ptr(), host, _stream(stream))
    if st not in (OK, 7):
        _check("pga_validate_inputs", st)
    return st, list(host)
