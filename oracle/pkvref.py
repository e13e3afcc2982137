"""ctypes wrapper over the C oracle (libpkvref.so).  Test infrastructure only.

Functions take torch CPU tensors (or numpy arrays) and return float64 numpy
arrays.  Argument marshalling only: all arithmetic is in pkvref.c.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

try:  # torch is optional for the wrapper; the workloads produce torch tensors
    import torch
except Exception:  # pragma: no cover
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkvref.so")
_lib = None

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3, "fp8_e5m2": 4}


def _configure(L):
    vp, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    L.pkvref_kv_append.argtypes = [C.c_int, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32]
    L.pkvref_gather.argtypes = [C.c_int, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    L.pkvref_decode.argtypes = [C.c_int, i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, i32,
                                vp, f32, vp, i64, vp, vp, i32]
    L.pkvref_prefill.argtypes = [C.c_int, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, vp,
                                 i32, vp, f32, vp, i64, vp, vp, i32]
    L.pkvref_decode_ex.argtypes = [C.c_int, C.c_int, i32, i32, i32, i32, vp, vp, f32, f32, vp,
                                   i32, i32, vp, i32, vp, f32, i32, i32, vp, i64, vp, vp, i32]
    L.pkvref_prefill_ex.argtypes = [C.c_int, C.c_int, i32, i32, i32, i32, vp, vp, f32, f32, vp,
                                    vp, i32, i32, vp, i32, vp, f32, vp, i64, vp, vp, i32]
    L.pkvref_merge.argtypes = [vp, vp, i64, i32, i32, vp, vp]
    L.pkvref_to_double.argtypes = [C.c_int, vp, i64, vp]
    L.pkvref_quant_fp8.argtypes = [C.c_int, C.c_int, vp, i64, f32, vp]
    for fn in ("pkvref_kv_append", "pkvref_gather", "pkvref_decode", "pkvref_prefill",
               "pkvref_merge", "pkvref_to_double", "pkvref_decode_ex", "pkvref_quant_fp8",
               "pkvref_prefill_ex"):
        getattr(L, fn).restype = C.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _configure(C.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Run the wrappers against another build of pkvref.c (used by the tests
    that plant a mistake in a copy of the oracle and check the pins catch it)."""
    global _lib
    saved = lib()
    _lib = _configure(C.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _ptr(x):
    """Host pointer of a contiguous torch CPU tensor or numpy array (None -> NULL)."""
    if x is None:
        return None
    if torch is not None and isinstance(x, torch.Tensor):
        assert x.device.type == "cpu" and x.is_contiguous(), "oracle takes contiguous CPU tensors"
        return x.data_ptr()
    assert isinstance(x, np.ndarray) and x.flags["C_CONTIGUOUS"]
    return x.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid argument or index out of range (rc={rc})")


def _i32(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.to(torch.int32).contiguous()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _rows(rows: Optional[Sequence[int]]):
    if rows is None:
        return None
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def kv_append(dtype: str, k_cache, v_cache, k_new, v_new, slots) -> None:
    """In place on the host pools: bitwise copy of each new token's K/V rows
    into page slot // P at offset slot % P (slot < 0 skipped)."""
    num_pages, hkv, p, d = k_cache.shape
    slots = _i32(slots)
    n = int(slots.shape[0])
    _check(lib().pkvref_kv_append(DTYPE_CODES[dtype], num_pages, p, hkv, d, _ptr(k_cache),
                                  _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(slots), n),
           "kv_append")


def gather(dtype: str, k_cache, v_cache, table_row, length: int):
    """Logical tokens [0, length) of one sequence as contiguous [L][H_kv][D]
    tensors of the cache dtype (bitwise)."""
    num_pages, hkv, p, d = k_cache.shape
    table_row = _i32(table_row)
    k_out = torch.empty((length, hkv, d), dtype=k_cache.dtype)
    v_out = torch.empty_like(k_out)
    _check(lib().pkvref_gather(DTYPE_CODES[dtype], num_pages, p, hkv, d, _ptr(k_cache),
                               _ptr(v_cache), _ptr(table_row), int(length), _ptr(k_out),
                               _ptr(v_out)), "gather")
    return k_out, v_out


def decode(dtype: str, k_cache, v_cache, q, block_table, context_lens, scale: float,
           rows: Optional[Sequence[int]] = None, n_threads: int = 0):
    """Decode attention.  Returns (out [n_rows][D], lse [n_rows]) in float64;
    rows are indices b * H_q + h (default: all, in order)."""
    num_pages, hkv, p, d = k_cache.shape
    batch, hq, dq = q.shape
    assert dq == d
    bt = _i32(block_table)
    cl = _i32(context_lens)
    r = _rows(rows)
    n = batch * hq if r is None else int(r.shape[0])
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    _check(lib().pkvref_decode(DTYPE_CODES[dtype], num_pages, p, hkv, d, _ptr(k_cache),
                               _ptr(v_cache), _ptr(q), batch, hq, _ptr(bt), int(bt.shape[1]),
                               _ptr(cl), float(scale), _ptr(r), n, _ptr(out), _ptr(lse),
                               int(n_threads)), "decode")
    return out, lse


def decode_ex(q_dtype: str, kv_dtype: str, k_cache, v_cache, q, block_table, context_lens,
              scale: float, k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0,
              sink: int = 0, rows: Optional[Sequence[int]] = None, n_threads: int = 0):
    """Decode attention with a cache type apart from the query type (fp8 pools
    with per-tensor scales) and an optional sliding window: with window > 0
    the query sees keys t >= L - window and t < sink.  Returns (out, lse) in
    float64 as decode() does."""
    num_pages, hkv, p, d = k_cache.shape
    batch, hq, dq = q.shape
    assert dq == d
    bt = _i32(block_table)
    cl = _i32(context_lens)
    r = _rows(rows)
    n = batch * hq if r is None else int(r.shape[0])
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    _check(lib().pkvref_decode_ex(DTYPE_CODES[q_dtype], DTYPE_CODES[kv_dtype], num_pages, p, hkv,
                                  d, _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                  float(v_scale), _ptr(q), batch, hq, _ptr(bt), int(bt.shape[1]),
                                  _ptr(cl), float(scale), int(window), int(sink), _ptr(r), n,
                                  _ptr(out), _ptr(lse), int(n_threads)), "decode_ex")
    return out, lse


def quant_fp8(fp8_dtype: str, src_dtype: str, x, scale: float) -> np.ndarray:
    """fp8 codes (uint8, same shape) of x / scale: the division in fp32, the
    nearest code with ties to the even one, clipped to the largest finite
    value; NaN gives 0x7F."""
    x = x.contiguous() if torch is not None and isinstance(x, torch.Tensor) else x
    n = int(np.prod(x.shape))
    out = np.zeros(tuple(x.shape), dtype=np.uint8)
    _check(lib().pkvref_quant_fp8(DTYPE_CODES[fp8_dtype], DTYPE_CODES[src_dtype], _ptr(x), n,
                                  float(scale), _ptr(out)), "quant_fp8")
    return out


def prefill(dtype: str, k_cache, v_cache, q, q_indptr, block_table, kv_lens, scale: float,
            rows: Optional[Sequence[int]] = None, n_threads: int = 0):
    """Chunked-prefill attention over the cache.  q packed [sum C][H_q][D].
    Returns (out [n_rows][D], lse [n_rows]) in float64; rows are indices
    tok * H_q + h (default: all)."""
    return prefill_ex(dtype, dtype, k_cache, v_cache, q, q_indptr, block_table, kv_lens, scale,
                      rows=rows, n_threads=n_threads)


def prefill_ex(q_dtype: str, kv_dtype: str, k_cache, v_cache, q, q_indptr, block_table, kv_lens,
               scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
               rows: Optional[Sequence[int]] = None, n_threads: int = 0):
    """Chunked prefill over a cache type apart from the query type (fp8 pools
    with per-tensor scales).  Returns (out, lse) in float64 as prefill()."""
    num_pages, hkv, p, d = k_cache.shape
    n_tok, hq, dq = q.shape
    assert dq == d
    qi = _i32(q_indptr)
    batch = int(qi.shape[0]) - 1
    bt = _i32(block_table)
    kl = _i32(kv_lens)
    r = _rows(rows)
    n = n_tok * hq if r is None else int(r.shape[0])
    out = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    _check(lib().pkvref_prefill_ex(DTYPE_CODES[q_dtype], DTYPE_CODES[kv_dtype], num_pages, p,
                                   hkv, d, _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                   float(v_scale), _ptr(q), _ptr(qi), batch, hq, _ptr(bt),
                                   int(bt.shape[1]), _ptr(kl), float(scale), _ptr(r), n,
                                   _ptr(out), _ptr(lse), int(n_threads)), "prefill_ex")
    return out, lse


def merge(o_parts, lse_parts):
    """Merge partial states.  o_parts [rows][n][D], lse_parts [rows][n]
    (float64 or convertible).  Returns (out [rows][D], lse [rows])."""
    o = np.ascontiguousarray(np.asarray(o_parts, dtype=np.float64))
    l = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
    rows, n, d = o.shape
    out = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    _check(lib().pkvref_merge(_ptr(o), _ptr(l), rows, n, d, _ptr(out), _ptr(lse)), "merge")
    return out, lse


def to_double(dtype: str, x) -> np.ndarray:
    """Exact widening of a tensor of the given element type to float64."""
    x = x.contiguous() if torch is not None and isinstance(x, torch.Tensor) else x
    n = int(np.prod(x.shape))
    out = np.zeros(tuple(x.shape), dtype=np.float64)
    _check(lib().pkvref_to_double(DTYPE_CODES[dtype], _ptr(x), n, _ptr(out)), "to_double")
    return out
