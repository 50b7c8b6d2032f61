"""fp64 CPU oracle for paged GQA attention (head_dim 256).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The library path never imports this
package, and this package never imports the library.  Both read their inputs
from ``workloads``, which only draws random numbers.

The arithmetic lives in ``oracle.cpp`` (plain fp64 C++ with OpenMP); this
module builds it with g++ and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_handle = None

_DTYPE = {"bf16": 1, "fp8_e4m3": 2}


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so next to it."""
    if not force and os.path.exists(_SO):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


class _KV(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("k_stride_page", ctypes.c_int64), ("k_stride_token", ctypes.c_int64), ("k_stride_head", ctypes.c_int64),
        ("v_stride_page", ctypes.c_int64), ("v_stride_token", ctypes.c_int64), ("v_stride_head", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
        ("k_descale", ctypes.c_double), ("v_descale", ctypes.c_double),
    ]


def _lib():
    global _handle
    with _lock:
        if _handle is None:
            if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
                build()
            h = ctypes.CDLL(_SO)
            P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
            h.oracle_causal_attention.argtypes = [P, I32, D, I32, I32, P, P, ctypes.POINTER(_KV), D, P, I64, P, P, I32]
            h.oracle_causal_attention.restype = ctypes.c_int
            h.oracle_sparse_attention.argtypes = [P, I32, D, I32, I32, P, P, P, I64, I32, ctypes.POINTER(_KV), D,
                                                  P, I64, P, P, I32]
            h.oracle_sparse_attention.restype = ctypes.c_int
            h.oracle_causal_probs.argtypes = [P, I32, D, I32, I32, P, P, ctypes.POINTER(_KV), D, I64, I32, P]
            h.oracle_causal_probs.restype = ctypes.c_int
            h.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
            h.oracle_decode_bf16.restype = D
            h.oracle_decode_e4m3fn.argtypes = [ctypes.c_uint8]
            h.oracle_decode_e4m3fn.restype = D
            h.oracle_encode_e4m3fn.argtypes = [ctypes.c_float]
            h.oracle_encode_e4m3fn.restype = ctypes.c_uint8
            h.oracle_quantize_fp8.argtypes = [P, I64, P, P, P]
            h.oracle_quantize_fp8.restype = ctypes.c_int
            h.oracle_write_new_kv.argtypes = [P, P, I32, P, P, ctypes.POINTER(_KV), ctypes.c_float, ctypes.c_float]
            h.oracle_write_new_kv.restype = ctypes.c_int
            _handle = h
    return _handle


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _kv(p) -> _KV:
    ks = p.kv_strides()
    kv = _KV()
    kv.k_cache, kv.v_cache = _ptr(p.k_cache), _ptr(p.v_cache)
    kv.dtype = _DTYPE[p.kv_dtype]
    kv.num_kv_heads, kv.head_dim, kv.page_size = p.num_kv_heads, p.head_dim, p.page_size
    kv.num_pages = p.num_pages
    kv.k_stride_page, kv.k_stride_token, kv.k_stride_head = ks
    kv.v_stride_page, kv.v_stride_token, kv.v_stride_head = ks
    kv.block_table = _ptr(p.block_table)
    kv.block_table_stride = p.block_table.shape[1]
    kv.k_descale, kv.v_descale = float(p.k_descale), float(p.v_descale)
    return kv


def attention(p, rows=None, threads: int = 0):
    """fp64 (out [T, Hq, 256], lse [T, Hq]) of problem ``p``.  With ``rows`` (an
    array of query-token indices) only those rows are computed; the rest are NaN."""
    h = _lib()
    T, Hq = p.num_tokens, p.num_q_heads
    out = np.full((T, Hq, p.head_dim), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    kv = _kv(p)
    cu = np.ascontiguousarray(p.cu_seqlens_q, dtype=np.int32)
    lk = np.ascontiguousarray(p.seq_lens_k, dtype=np.int32)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nr = _ptr(rows), rows.size
    else:
        rp, nr = None, 0
    if p.mode == "sparse":
        idx = np.ascontiguousarray(p.indices, dtype=np.int32)
        rc = h.oracle_sparse_attention(_ptr(p.q), _DTYPE[p.q_dtype], float(p.q_descale), Hq, p.num_seqs,
                                       _ptr(cu), _ptr(lk), _ptr(idx), idx.shape[1], idx.shape[1],
                                       ctypes.byref(kv), float(p.softmax_scale), rp, nr, _ptr(out), _ptr(lse),
                                       threads)
    else:
        rc = h.oracle_causal_attention(_ptr(p.q), _DTYPE[p.q_dtype], float(p.q_descale), Hq, p.num_seqs,
                                       _ptr(cu), _ptr(lk), ctypes.byref(kv), float(p.softmax_scale), rp, nr,
                                       _ptr(out), _ptr(lse), threads)
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    return out, lse


def causal_probs(p, token: int, head: int) -> np.ndarray:
    """Normalised weights of (token, head) over keys 0..Lk_b-1 (0 where masked)."""
    h = _lib()
    b = int(np.searchsorted(p.cu_seqlens_q, token, side="right") - 1)
    probs = np.full(int(p.seq_lens_k[b]), np.nan)
    kv = _kv(p)
    cu = np.ascontiguousarray(p.cu_seqlens_q, dtype=np.int32)
    lk = np.ascontiguousarray(p.seq_lens_k, dtype=np.int32)
    rc = h.oracle_causal_probs(_ptr(p.q), _DTYPE[p.q_dtype], float(p.q_descale), p.num_q_heads, p.num_seqs,
                               _ptr(cu), _ptr(lk), ctypes.byref(kv), float(p.softmax_scale), token, head,
                               _ptr(probs))
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    return probs


def decode_bf16(bits: int) -> float:
    return _lib().oracle_decode_bf16(bits)


def decode_e4m3fn(code: int) -> float:
    return _lib().oracle_decode_e4m3fn(code)


def encode_e4m3fn(y: float) -> int:
    """E4M3FN code nearest to the fp32 value ``y`` (ties to even, saturating)."""
    return int(_lib().oracle_encode_e4m3fn(float(np.float32(y))))


def quantize_fp8(x_bits: np.ndarray, descale=None):
    """Per-tensor FP8 quantisation of bf16 patterns ``x_bits`` (any shape).

    ``descale=None`` takes the dynamic scale amax/448; otherwise the given fp32
    descale.  Returns (uint8 codes of the same shape, fp32 descale)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.empty(x.shape, dtype=np.uint8)
    out = np.zeros(1, dtype=np.float32)
    din = None if descale is None else np.array([descale], dtype=np.float32)
    rc = _lib().oracle_quantize_fp8(_ptr(x), x.size, None if din is None else _ptr(din), _ptr(codes), _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the quantisation (code %d)" % rc)
    return codes, float(out[0])


def write_new_kv(p, k_new: np.ndarray, v_new: np.ndarray, cu_seqlens_k: np.ndarray) -> None:
    """Quantise the new tokens' keys and values (bf16 [T, Hkv, 256]) with the
    pool's descales of problem ``p`` and write them into ``p``'s FP8 pools in
    place, at logical positions Lk_b - Lq_b + t."""
    k = np.ascontiguousarray(k_new, dtype=np.uint16)
    v = np.ascontiguousarray(v_new, dtype=np.uint16)
    cu_q = np.ascontiguousarray(p.cu_seqlens_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    assert p.k_cache.flags["C_CONTIGUOUS"] and p.v_cache.flags["C_CONTIGUOUS"]
    kv = _kv(p)
    rc = _lib().oracle_write_new_kv(_ptr(k), _ptr(v), p.num_seqs, _ptr(cu_q), _ptr(cu_k), ctypes.byref(kv),
                                    float(np.float32(p.k_descale)), float(np.float32(p.v_descale)))
    if rc != 0:
        raise ValueError("oracle rejected the key/value write (code %d)" % rc)


def quantized_problem(p):
    """The oracle's FP8 quantisation of a quantising prefill problem (one whose
    ``meta`` holds bf16 ``k_new`` / ``v_new``): a copy whose Q holds the FP8
    codes under the dynamic descale and whose pool holds the new keys and
    values, ready for :func:`attention`."""
    import copy

    r = copy.copy(p)
    r.k_cache, r.v_cache = p.k_cache.copy(), p.v_cache.copy()
    r.q, r.q_descale = quantize_fp8(p.q)
    r.q_dtype = "fp8_e4m3"
    write_new_kv(r, p.meta["k_new"], p.meta["v_new"], p.meta["cu_seqlens_k"])
    r.meta = {k: v for k, v in p.meta.items() if k not in ("k_new", "v_new")}
    return r

