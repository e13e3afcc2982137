"""Thin ctypes binding over libpkv.so (include/pkv.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  If the
library is not built the first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pkv.h")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_FP8_E5M2 = 0, 1, 2, 3, 4
_TORCH_TO_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
                  torch.float8_e4m3fn: PKV_FP8_E4M3, torch.float8_e5m2: PKV_FP8_E5M2}
_CODE_TO_TORCH = {v: k for k, v in _TORCH_TO_CODE.items()}
_FP8 = (torch.float8_e4m3fn, torch.float8_e5m2)
STATUS = {0: "PKV_OK", -1: "PKV_ERR_INVALID", -2: "PKV_ERR_UNSUPPORTED",
          -3: "PKV_ERR_WORKSPACE", -4: "PKV_ERR_HIP"}


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class CacheDesc(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32)]


class DecodeOpts(C.Structure):
    _fields_ = [("q_dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
                ("window", C.c_int32), ("sink", C.c_int32)]


_lib = None


def lib():
    """Load libpkv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32, f32, sz = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
        dp = C.POINTER(CacheDesc)
        L.pkv_version.restype = C.c_int
        L.pkv_last_error.restype = C.c_char_p
        L.pkv_kv_append.argtypes = [dp, vp, vp, vp, vp, vp, i32, vp]
        L.pkv_gather_kv.argtypes = [dp, vp, vp, vp, i32, vp, vp, vp]
        L.pkv_decode_plan.argtypes = [dp, i32, i32, i32, i32, C.POINTER(i32), C.POINTER(sz)]
        L.pkv_paged_attn_decode.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp, i32, f32, i32,
                                            vp, vp, vp, sz, vp]
        L.pkv_paged_attn_decode_partials.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp, i32,
                                                     f32, i32, vp, sz, vp]
        L.pkv_merge_states.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.pkv_paged_attn_prefill_chunk.argtypes = [dp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                   i32, vp, i32, f32, vp, vp, vp]
        L.pkv_validate_tables.argtypes = [dp, vp, i32, vp, i32, vp, i32]
        op = C.POINTER(DecodeOpts)
        L.pkv_decode_plan_ex.argtypes = [dp, i32, i32, i32, i32, op, C.POINTER(i32),
                                         C.POINTER(sz)]
        L.pkv_paged_attn_decode_ex.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp, i32, f32,
                                               i32, op, vp, vp, vp, sz, vp]
        L.pkv_paged_attn_decode_partials_ex.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp,
                                                        i32, f32, i32, op, vp, sz, vp]
        L.pkv_kv_append_quant.argtypes = [dp, vp, vp, vp, vp, i32, f32, f32, vp, i32, vp]
        L.pkv_paged_attn_mixed.argtypes = [dp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32,
                                           vp, i32, f32, i32, vp, vp, vp, sz, vp]
        L.pkv_decode_split_for_lens.argtypes = [dp, i32, i32, vp, op, C.POINTER(i32)]
        L.pkv_paged_attn_prefill_chunk_ex.argtypes = [dp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                      vp, i32, vp, i32, f32, op, vp, vp, vp]
        L.pkv_paged_attn_mixed_ex.argtypes = [dp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp,
                                              i32, vp, i32, f32, i32, op, vp, vp, vp, sz, vp]
        L.pkv_decode_shared_prefix_plan.argtypes = [dp, i32, i32, i32, i32, i32, op,
                                                    C.POINTER(i32), C.POINTER(sz)]
        L.pkv_paged_attn_decode_shared_prefix.argtypes = [dp, vp, vp, vp, i32, i32, vp, i32, vp,
                                                          i32, vp, i32, f32, i32, op, vp, vp, vp,
                                                          sz, vp]
        L.pkv_paged_attn_decode_append.argtypes = [dp, vp, vp, vp, vp, vp, i32, i32, vp, i32,
                                                   vp, i32, f32, i32, op, vp, vp, vp, sz, vp]
        L.pkv_paged_attn_decode_append_partials.argtypes = [dp, vp, vp, vp, vp, vp, i32, i32,
                                                            vp, i32, vp, i32, f32, i32, op, vp,
                                                            sz, vp]
        L.pkv_paged_attn_decode_append_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, i32, i32,
                                                           vp, i32, vp, i32, f32, i32, op, vp,
                                                           vp, vp]
        L.pkv_noalloc_scratch_bytes.restype = sz
        L.pkv_noalloc_scratch_bytes.argtypes = []
        L.pkv_probe_read.argtypes = [vp, sz, vp, i32, i32, vp, vp]
        L.pkv_probe_mfma.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.pkv_probe_prefill_loop.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        for name in ("pkv_kv_append", "pkv_gather_kv", "pkv_decode_plan", "pkv_paged_attn_decode",
                     "pkv_paged_attn_decode_partials", "pkv_merge_states",
                     "pkv_paged_attn_prefill_chunk", "pkv_validate_tables",
                     "pkv_decode_plan_ex", "pkv_paged_attn_decode_ex",
                     "pkv_paged_attn_decode_partials_ex", "pkv_kv_append_quant",
                     "pkv_paged_attn_mixed", "pkv_decode_split_for_lens",
                     "pkv_paged_attn_prefill_chunk_ex", "pkv_paged_attn_mixed_ex",
                     "pkv_decode_shared_prefix_plan", "pkv_paged_attn_decode_shared_prefix",
                     "pkv_paged_attn_decode_append", "pkv_paged_attn_decode_append_partials",
                     "pkv_paged_attn_decode_append_noalloc", "pkv_probe_read",
                     "pkv_probe_mfma", "pkv_probe_prefill_loop"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def declared_symbols():
    """Names of the functions include/pkv.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def _check(rc: int):
    if rc != 0:
        raise PkvError(rc, lib().pkv_last_error().decode())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    """Descriptor of a [num_pages][H_kv][P][D] pool."""
    if k_cache.dim() != 4:
        raise ValueError("cache must be [num_pages][num_kv_heads][page_size][head_dim]")
    if k_cache.dtype not in _TORCH_TO_CODE:
        raise TypeError(f"unsupported cache dtype {k_cache.dtype}")
    n, h, p, d = k_cache.shape
    return CacheDesc(n, p, h, d, _TORCH_TO_CODE[k_cache.dtype])


def _check_pools(k_cache, v_cache):
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache", k_cache.dtype)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    return cache_desc(k_cache)


def kv_append(k_cache, v_cache, k_new, v_new, slots) -> None:
    """pkv_kv_append: store new tokens' K/V rows [n][H_kv][D] at their slots."""
    desc = _check_pools(k_cache, v_cache)
    _dev(k_new, "k_new", k_cache.dtype)
    _dev(v_new, "v_new", k_cache.dtype)
    _dev(slots, "slots", torch.int32)
    n = int(slots.shape[0])
    if k_new.shape != (n, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [n][H_kv][D]")
    _check(lib().pkv_kv_append(C.byref(desc), _p(k_cache), _p(v_cache), _p(k_new), _p(v_new),
                               _p(slots), n, _stream()))


def gather_kv(k_cache, v_cache, table_row, length: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """pkv_gather_kv: logical tokens [0, length) as contiguous [L][H_kv][D]."""
    desc = _check_pools(k_cache, v_cache)
    _dev(table_row, "table_row", torch.int32)
    k_out = torch.empty((length, desc.num_kv_heads, desc.head_dim), dtype=k_cache.dtype,
                        device=k_cache.device)
    v_out = torch.empty_like(k_out)
    _check(lib().pkv_gather_kv(C.byref(desc), _p(k_cache), _p(v_cache), _p(table_row),
                               int(length), _p(k_out), _p(v_out), _stream()))
    return k_out, v_out


def kv_append_quant(k_cache, v_cache, k_new, v_new, slots, k_scale: float,
                    v_scale: float) -> None:
    """pkv_kv_append_quant: quantize new tokens' K/V rows [n][H_kv][D] (f32,
    f16 or bf16) into an fp8 cache at their slots."""
    desc = _check_pools(k_cache, v_cache)
    if k_cache.dtype not in _FP8:
        raise TypeError("kv_append_quant writes fp8 caches")
    _dev(k_new, "k_new")
    _dev(v_new, "v_new", k_new.dtype)
    _dev(slots, "slots", torch.int32)
    n = int(slots.shape[0])
    if k_new.shape != (n, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [n][H_kv][D]")
    _check(lib().pkv_kv_append_quant(C.byref(desc), _p(k_cache), _p(v_cache), _p(k_new),
                                     _p(v_new), _TORCH_TO_CODE[k_new.dtype], float(k_scale),
                                     float(v_scale), _p(slots), n, _stream()))


def decode_opts(q_dtype: torch.dtype, k_cache_dtype: torch.dtype, k_scale: float = 1.0,
                v_scale: float = 1.0, window: int = 0, sink: int = 0) -> Optional[DecodeOpts]:
    """pkv_decode_opts for the *_ex calls, or None when every option has its
    default (plain calls)."""
    if (q_dtype == k_cache_dtype and k_scale == 1.0 and v_scale == 1.0 and window == 0
            and sink == 0):
        return None
    return DecodeOpts(_TORCH_TO_CODE[q_dtype], float(k_scale), float(v_scale), int(window),
                      int(sink))


def decode_plan(desc: CacheDesc, batch: int, num_q_heads: int, max_context_len: int,
                split_tokens: int = 0, opts: Optional[DecodeOpts] = None) -> Tuple[int, int]:
    """pkv_decode_plan (pkv_decode_plan_ex with options): (n_split, workspace_bytes)."""
    n = C.c_int32(0)
    ws = C.c_size_t(0)
    if opts is None:
        _check(lib().pkv_decode_plan(C.byref(desc), int(batch), int(num_q_heads),
                                     int(max_context_len), int(split_tokens), C.byref(n),
                                     C.byref(ws)))
    else:
        _check(lib().pkv_decode_plan_ex(C.byref(desc), int(batch), int(num_q_heads),
                                        int(max_context_len), int(split_tokens), C.byref(opts),
                                        C.byref(n), C.byref(ws)))
    return int(n.value), int(ws.value)


def decode_split_for_lens(desc: CacheDesc, num_q_heads: int, lens,
                          opts: Optional[DecodeOpts] = None) -> int:
    """pkv_decode_split_for_lens: split_tokens for a batch of known lengths
    (a sequence of ints or a CPU int tensor)."""
    ln = torch.as_tensor(lens, dtype=torch.int32).contiguous().cpu()
    out = C.c_int32(0)
    _check(lib().pkv_decode_split_for_lens(C.byref(desc), int(ln.numel()), int(num_q_heads),
                                           _p(ln) if ln.numel() else None,
                                           C.byref(opts) if opts is not None else None,
                                           C.byref(out)))
    return int(out.value)


def partials_bytes(batch: int, num_q_heads: int, n_split: int, head_dim: int) -> Tuple[int, int]:
    """(o_bytes rounded to 256, total) of the partials layout in include/pkv.h."""
    rows = batch * num_q_heads
    ob = rows * n_split * head_dim * 4
    ob = (ob + 255) & ~255
    return ob, ob + rows * n_split * 4


def _decode_common(q, k_cache, v_cache, block_table, context_lens, max_context_len):
    desc = _check_pools(k_cache, v_cache)
    if k_cache.dtype in _FP8:
        _dev(q, "q")
        if q.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError("queries over an fp8 cache must be float16 or bfloat16")
    else:
        _dev(q, "q", k_cache.dtype)
    _dev(block_table, "block_table", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B][H_q][D]")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    if block_table.dim() != 2 or block_table.shape[0] != batch or context_lens.shape != (batch,):
        raise ValueError("block_table must be [B][stride] and context_lens [B]")
    return desc, batch, hq


def paged_attn_decode(q, k_cache, v_cache, block_table, context_lens, max_context_len: int,
                      scale: float, split_tokens: int = 0, out=None, lse_out=None,
                      workspace=None, return_lse: bool = False, k_scale: float = 1.0,
                      v_scale: float = 1.0, window: int = 0, sink: int = 0):
    """pkv_paged_attn_decode (pkv_paged_attn_decode_ex when an fp8 cache, its
    scales or a window are given).  Returns out [B][H_q][D] in q's dtype (and
    lse [B][H_q])."""
    desc, batch, hq = _decode_common(q, k_cache, v_cache, block_table, context_lens,
                                     max_context_len)
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale, window, sink)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse_out is None:
        lse_out = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    n_split, ws_bytes = decode_plan(desc, batch, hq, max_context_len, split_tokens, opts)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    common = (C.byref(desc), _p(k_cache), _p(v_cache), _p(q), batch, hq, _p(block_table),
              int(block_table.shape[1]), _p(context_lens), int(max_context_len), float(scale),
              int(split_tokens))
    tail = (_p(out), _p(lse_out), _p(workspace), ws_len, _stream())
    if opts is None:
        _check(lib().pkv_paged_attn_decode(*common, *tail))
    else:
        _check(lib().pkv_paged_attn_decode_ex(*common, C.byref(opts), *tail))
    return (out, lse_out) if return_lse else out


def paged_attn_decode_partials(q, k_cache, v_cache, block_table, context_lens,
                               max_context_len: int, scale: float, split_tokens: int = 0,
                               workspace=None, k_scale: float = 1.0, v_scale: float = 1.0,
                               window: int = 0, sink: int = 0):
    """pkv_paged_attn_decode_partials (or its _ex form).  Returns (o_parts
    [B*H_q][n][D], lse_parts [B*H_q][n], workspace) as views of the
    workspace."""
    desc, batch, hq = _decode_common(q, k_cache, v_cache, block_table, context_lens,
                                     max_context_len)
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale, window, sink)
    n_split, _ = decode_plan(desc, batch, hq, max_context_len, split_tokens, opts)
    ob, total = partials_bytes(batch, hq, n_split, desc.head_dim)
    if workspace is None:
        workspace = torch.empty(total, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size()
    common = (C.byref(desc), _p(k_cache), _p(v_cache), _p(q), batch, hq, _p(block_table),
              int(block_table.shape[1]), _p(context_lens), int(max_context_len), float(scale),
              int(split_tokens))
    if opts is None:
        _check(lib().pkv_paged_attn_decode_partials(*common, _p(workspace), ws_len, _stream()))
    else:
        _check(lib().pkv_paged_attn_decode_partials_ex(*common, C.byref(opts), _p(workspace),
                                                       ws_len, _stream()))
    rows = batch * hq
    o_parts = workspace[:rows * n_split * desc.head_dim * 4].view(torch.float32).view(
        rows, n_split, desc.head_dim)
    lse_parts = workspace[ob:ob + rows * n_split * 4].view(torch.float32).view(rows, n_split)
    return o_parts, lse_parts, workspace


def _append_common(q, k_cache, v_cache, k_new, v_new, block_table, context_lens,
                   max_context_len, scale, split_tokens, k_scale, v_scale, window, sink):
    """Checks and the leading C arguments shared by the decode-with-append calls."""
    desc, batch, hq = _decode_common(q, k_cache, v_cache, block_table, context_lens,
                                     max_context_len)
    _dev(k_new, "k_new", q.dtype)
    _dev(v_new, "v_new", q.dtype)
    if (k_new.shape != (batch, desc.num_kv_heads, desc.head_dim)
            or v_new.shape != k_new.shape):
        raise ValueError("k_new/v_new must be [B][H_kv][D]")
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale, window, sink)
    common = (C.byref(desc), _p(k_cache), _p(v_cache), _p(k_new), _p(v_new), _p(q), batch, hq,
              _p(block_table), int(block_table.shape[1]), _p(context_lens),
              int(max_context_len), float(scale), int(split_tokens),
              C.byref(opts) if opts is not None else None)
    return desc, batch, hq, opts, common


def paged_attn_decode_append(q, k_cache, v_cache, k_new, v_new, block_table, context_lens,
                             max_context_len: int, scale: float, split_tokens: int = 0,
                             out=None, lse_out=None, workspace=None, return_lse: bool = False,
                             k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0,
                             sink: int = 0):
    """pkv_paged_attn_decode_append: stores k_new[b] / v_new[b] ([B][H_kv][D],
    q's dtype) at position context_lens[b] - 1 of each sequence (quantized by
    the scales for fp8 caches) and decodes, in the decode's own launches.
    Returns out (and lse) as paged_attn_decode does."""
    desc, batch, hq, opts, common = _append_common(
        q, k_cache, v_cache, k_new, v_new, block_table, context_lens, max_context_len, scale,
        split_tokens, k_scale, v_scale, window, sink)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse_out is None:
        lse_out = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    _, ws_bytes = decode_plan(desc, batch, hq, max_context_len, split_tokens, opts)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_append(*common, _p(out), _p(lse_out), _p(workspace),
                                              ws_len, _stream()))
    return (out, lse_out) if return_lse else out


def paged_attn_decode_append_noalloc(q, k_cache, v_cache, k_new, v_new, block_table,
                                     context_lens, max_context_len: int, scale: float,
                                     split_tokens: int = 0, out=None, lse_out=None,
                                     return_lse: bool = False, k_scale: float = 1.0,
                                     v_scale: float = 1.0, window: int = 0, sink: int = 0):
    """pkv_paged_attn_decode_append_noalloc: paged_attn_decode_append with its
    split partials in the library's static device array instead of a
    workspace.  out and lse_out are the caller's (allocated here only when
    not given)."""
    desc, batch, hq, opts, common = _append_common(
        q, k_cache, v_cache, k_new, v_new, block_table, context_lens, max_context_len, scale,
        split_tokens, k_scale, v_scale, window, sink)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse_out is None:
        lse_out = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    _check(lib().pkv_paged_attn_decode_append_noalloc(*common, _p(out), _p(lse_out), _stream()))
    return (out, lse_out) if return_lse else out


def noalloc_scratch_bytes() -> int:
    """Size of the static scratch array of paged_attn_decode_append_noalloc."""
    return int(lib().pkv_noalloc_scratch_bytes())


def paged_attn_decode_append_partials(q, k_cache, v_cache, k_new, v_new, block_table,
                                      context_lens, max_context_len: int, scale: float,
                                      split_tokens: int = 0, workspace=None,
                                      k_scale: float = 1.0, v_scale: float = 1.0,
                                      window: int = 0, sink: int = 0):
    """pkv_paged_attn_decode_append_partials: the append and the first pass.
    Returns (o_parts, lse_parts, workspace) as paged_attn_decode_partials."""
    desc, batch, hq, opts, common = _append_common(
        q, k_cache, v_cache, k_new, v_new, block_table, context_lens, max_context_len, scale,
        split_tokens, k_scale, v_scale, window, sink)
    n_split, _ = decode_plan(desc, batch, hq, max_context_len, split_tokens, opts)
    ob, total = partials_bytes(batch, hq, n_split, desc.head_dim)
    if workspace is None:
        workspace = torch.empty(total, dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_append_partials(*common, _p(workspace), ws_len,
                                                       _stream()))
    rows = batch * hq
    o_parts = workspace[:rows * n_split * desc.head_dim * 4].view(torch.float32).view(
        rows, n_split, desc.head_dim)
    lse_parts = workspace[ob:ob + rows * n_split * 4].view(torch.float32).view(rows, n_split)
    return o_parts, lse_parts, workspace


def merge_states(o_parts, lse_parts, out_dtype=torch.float32, out=None, lse_out=None,
                 return_lse: bool = False):
    """pkv_merge_states.  o_parts [rows][n][D] float32, lse_parts [rows][n]."""
    _dev(o_parts, "o_parts", torch.float32)
    _dev(lse_parts, "lse_parts", torch.float32)
    rows, n, d = (int(x) for x in o_parts.shape)
    if lse_parts.shape != (rows, n):
        raise ValueError("lse_parts must be [rows][n_parts]")
    if out is None:
        out = torch.empty((rows, d), dtype=out_dtype, device=o_parts.device)
    if return_lse and lse_out is None:
        lse_out = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    _check(lib().pkv_merge_states(_p(o_parts), _p(lse_parts), rows, n, d,
                                  _TORCH_TO_CODE[out.dtype], _p(out), _p(lse_out), _stream()))
    return (out, lse_out) if return_lse else out


def _query_type(q, k_cache):
    if k_cache.dtype in _FP8:
        _dev(q, "q")
        if q.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError("queries over an fp8 cache must be float16 or bfloat16")
    else:
        _dev(q, "q", k_cache.dtype)


def paged_attn_prefill_chunk(q, k_cache, v_cache, q_indptr, block_table, kv_lens,
                             max_q_len: int, max_kv_len: int, scale: float, out=None,
                             lse_out=None, return_lse: bool = False, k_scale: float = 1.0,
                             v_scale: float = 1.0):
    """pkv_paged_attn_prefill_chunk (pkv_paged_attn_prefill_chunk_ex for an fp8
    cache and its scales).  q packed [sum C][H_q][D]."""
    desc = _check_pools(k_cache, v_cache)
    _query_type(q, k_cache)
    _dev(q_indptr, "q_indptr", torch.int32)
    _dev(block_table, "block_table", torch.int32)
    _dev(kv_lens, "kv_lens", torch.int32)
    batch = int(q_indptr.shape[0]) - 1
    hq = int(q.shape[1])
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse_out is None:
        lse_out = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [sum C][H_q][D]")
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale)
    args = (C.byref(desc), _p(k_cache), _p(v_cache), _p(q), _p(q_indptr), batch, hq,
            int(q.shape[0]), int(max_q_len), _p(block_table), int(block_table.shape[1]),
            _p(kv_lens), int(max_kv_len), float(scale))
    tail = (_p(out), _p(lse_out), _stream())
    if opts is None:
        _check(lib().pkv_paged_attn_prefill_chunk(*args, *tail))
    else:
        _check(lib().pkv_paged_attn_prefill_chunk_ex(*args, C.byref(opts), *tail))
    return (out, lse_out) if return_lse else out


def paged_attn_mixed(q, k_cache, v_cache, q_indptr, block_table, kv_lens, num_decode: int,
                     max_q_len: int, max_kv_len: int, scale: float, split_tokens: int = 0,
                     out=None, lse_out=None, workspace=None, return_lse: bool = False,
                     k_scale: float = 1.0, v_scale: float = 1.0):
    """pkv_paged_attn_mixed (pkv_paged_attn_mixed_ex for an fp8 cache and its
    scales): a decode-first ragged batch (sequences 0 .. num_decode-1 one row
    each, then prefill chunks), q packed [sum C][H_q][D]."""
    desc = _check_pools(k_cache, v_cache)
    _query_type(q, k_cache)
    _dev(q_indptr, "q_indptr", torch.int32)
    _dev(block_table, "block_table", torch.int32)
    _dev(kv_lens, "kv_lens", torch.int32)
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [sum C][H_q][D]")
    batch = int(q_indptr.shape[0]) - 1
    hq = int(q.shape[1])
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse_out is None:
        lse_out = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale)
    ws_bytes = 0
    if num_decode > 0:
        _, ws_bytes = decode_plan(desc, num_decode, hq, max_kv_len, split_tokens, opts)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (C.byref(desc), _p(k_cache), _p(v_cache), _p(q), _p(q_indptr), batch, int(num_decode),
            hq, int(q.shape[0]), int(max_q_len), _p(block_table), int(block_table.shape[1]),
            _p(kv_lens), int(max_kv_len), float(scale), int(split_tokens))
    tail = (_p(out), _p(lse_out), _p(workspace), ws_len, _stream())
    if opts is None:
        _check(lib().pkv_paged_attn_mixed(*args, *tail))
    else:
        _check(lib().pkv_paged_attn_mixed_ex(*args, C.byref(opts), *tail))
    return (out, lse_out) if return_lse else out


def shared_prefix_plan(desc: CacheDesc, batch: int, num_q_heads: int, prefix_len: int,
                       max_suffix_len: int, split_tokens: int = 0,
                       opts: Optional[DecodeOpts] = None) -> Tuple[int, int]:
    """pkv_decode_shared_prefix_plan: (n_parts, workspace_bytes)."""
    n = C.c_int32(0)
    ws = C.c_size_t(0)
    _check(lib().pkv_decode_shared_prefix_plan(C.byref(desc), int(batch), int(num_q_heads),
                                               int(prefix_len), int(max_suffix_len),
                                               int(split_tokens),
                                               None if opts is None else C.byref(opts),
                                               C.byref(n), C.byref(ws)))
    return n.value, ws.value


def paged_attn_decode_shared_prefix(q, k_cache, v_cache, prefix_table, prefix_len: int,
                                    block_table, suffix_lens, max_suffix_len: int, scale: float,
                                    split_tokens: int = 0, out=None, lse_out=None,
                                    workspace=None, return_lse: bool = False,
                                    k_scale: float = 1.0, v_scale: float = 1.0):
    """pkv_paged_attn_decode_shared_prefix: decode of a batch whose sequences
    all begin with the pages of prefix_table (prefix_len keys, whole pages);
    block_table [B][*] (row stride taken from the tensor, so a column slice of
    a full table works) and suffix_lens [B] describe each sequence's own
    pages.  Returns out [B][H_q][D] (and lse [B][H_q])."""
    desc = _check_pools(k_cache, v_cache)
    _query_type(q, k_cache)
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B][H_q][D]")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    _dev(prefix_table, "prefix_table", torch.int32)
    _dev(suffix_lens, "suffix_lens", torch.int32)
    if (not isinstance(block_table, torch.Tensor) or block_table.device.type != "cuda"
            or block_table.dtype != torch.int32 or block_table.dim() != 2
            or block_table.shape[0] != batch or block_table.stride(1) != 1):
        raise ValueError("block_table must be a CUDA int32 [B][*] tensor with contiguous rows")
    if suffix_lens.shape != (batch,):
        raise ValueError("suffix_lens must be [B]")
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse_out is None:
        lse_out = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    _, ws_bytes = shared_prefix_plan(desc, batch, hq, prefix_len, max_suffix_len, split_tokens,
                                     opts)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_shared_prefix(
        C.byref(desc), _p(k_cache), _p(v_cache), _p(q), batch, hq, _p(prefix_table),
        int(prefix_len), _p(block_table), int(block_table.stride(0)), _p(suffix_lens),
        int(max_suffix_len), float(scale), int(split_tokens),
        None if opts is None else C.byref(opts), _p(out), _p(lse_out), _p(workspace), ws_len,
        _stream()))
    return (out, lse_out) if return_lse else out


def validate_tables(desc: CacheDesc, block_table, lens, slots=None) -> None:
    """pkv_validate_tables on host copies (CPU int32 tensors)."""
    bt = block_table.to(torch.int32).contiguous().cpu()
    ln = lens.to(torch.int32).contiguous().cpu()
    sl = None if slots is None else slots.to(torch.int32).contiguous().cpu()
    _check(lib().pkv_validate_tables(C.byref(desc), _p(bt), int(bt.shape[1]) if bt.dim() == 2 else 0,
                                     _p(ln), int(ln.shape[0]), _p(sl),
                                     0 if sl is None else int(sl.shape[0])))


class PreparedCall:
    """A library call with its arguments marshalled once (device pointers,
    sizes and the stream current at preparation).  Calling it performs only
    the C call; the tensors must stay alive and unchanged in shape."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep          # tensors whose storage the pointers refer to

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc)


def prepare_kv_append(k_cache, v_cache, k_new, v_new, slots) -> PreparedCall:
    desc = _check_pools(k_cache, v_cache)
    _dev(k_new, "k_new", k_cache.dtype)
    _dev(v_new, "v_new", k_cache.dtype)
    _dev(slots, "slots", torch.int32)
    n = int(slots.shape[0])
    if k_new.shape != (n, desc.num_kv_heads, desc.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [n][H_kv][D]")
    args = (C.byref(desc), _p(k_cache), _p(v_cache), _p(k_new), _p(v_new), _p(slots), n,
            _stream())
    return PreparedCall(lib().pkv_kv_append, args, (desc, k_cache, v_cache, k_new, v_new, slots))


def prepare_decode(q, k_cache, v_cache, block_table, context_lens, max_context_len: int,
                   scale: float, split_tokens: int, out, lse_out=None, workspace=None,
                   k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0,
                   sink: int = 0) -> PreparedCall:
    """pkv_paged_attn_decode (its _ex form with options) with its arguments
    marshalled once: one launch when the plan has one split, partials and
    merge otherwise (the workspace from decode_plan)."""
    desc, batch, hq = _decode_common(q, k_cache, v_cache, block_table, context_lens,
                                     max_context_len)
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale, window, sink)
    _dev(out, "out", q.dtype)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    common = (C.byref(desc), _p(k_cache), _p(v_cache), _p(q), batch, hq, _p(block_table),
              int(block_table.shape[1]), _p(context_lens), int(max_context_len), float(scale),
              int(split_tokens))
    tail = (_p(out), _p(lse_out), _p(workspace), ws_len, _stream())
    if opts is None:
        fn, args = lib().pkv_paged_attn_decode, common + tail
    else:
        fn, args = lib().pkv_paged_attn_decode_ex, common + (C.byref(opts),) + tail
    return PreparedCall(fn, args, (desc, opts, q, k_cache, v_cache, block_table, context_lens,
                                   out, lse_out, workspace))


def prepare_decode_partials(q, k_cache, v_cache, block_table, context_lens,
                            max_context_len: int, scale: float, split_tokens: int,
                            workspace, k_scale: float = 1.0, v_scale: float = 1.0,
                            window: int = 0, sink: int = 0) -> PreparedCall:
    desc, batch, hq = _decode_common(q, k_cache, v_cache, block_table, context_lens,
                                     max_context_len)
    opts = decode_opts(q.dtype, k_cache.dtype, k_scale, v_scale, window, sink)
    _dev(workspace, "workspace")
    ws_len = workspace.numel() * workspace.element_size()
    common = (C.byref(desc), _p(k_cache), _p(v_cache), _p(q), batch, hq, _p(block_table),
              int(block_table.shape[1]), _p(context_lens), int(max_context_len), float(scale),
              int(split_tokens))
    if opts is None:
        fn, args = lib().pkv_paged_attn_decode_partials, common + (_p(workspace), ws_len,
                                                                   _stream())
    else:
        fn = lib().pkv_paged_attn_decode_partials_ex
        args = common + (C.byref(opts), _p(workspace), ws_len, _stream())
    return PreparedCall(fn, args,
                        (desc, opts, q, k_cache, v_cache, block_table, context_lens, workspace))


def prepare_decode_append_partials(q, k_cache, v_cache, k_new, v_new, block_table,
                                   context_lens, max_context_len: int, scale: float,
                                   split_tokens: int, workspace, k_scale: float = 1.0,
                                   v_scale: float = 1.0, window: int = 0,
                                   sink: int = 0) -> PreparedCall:
    _dev(workspace, "workspace")
    desc, _, _, opts, common = _append_common(
        q, k_cache, v_cache, k_new, v_new, block_table, context_lens, max_context_len, scale,
        split_tokens, k_scale, v_scale, window, sink)
    ws_len = workspace.numel() * workspace.element_size()
    return PreparedCall(lib().pkv_paged_attn_decode_append_partials,
                        common + (_p(workspace), ws_len, _stream()),
                        (desc, opts, q, k_cache, v_cache, k_new, v_new, block_table,
                         context_lens, workspace))


def prepare_decode_append(q, k_cache, v_cache, k_new, v_new, block_table, context_lens,
                          max_context_len: int, scale: float, split_tokens: int, out,
                          lse_out=None, workspace=None, k_scale: float = 1.0,
                          v_scale: float = 1.0, window: int = 0,
                          sink: int = 0) -> PreparedCall:
    """pkv_paged_attn_decode_append with its arguments marshalled once (a
    single launch when the plan has one split)."""
    desc, _, _, opts, common = _append_common(
        q, k_cache, v_cache, k_new, v_new, block_table, context_lens, max_context_len, scale,
        split_tokens, k_scale, v_scale, window, sink)
    _dev(out, "out", q.dtype)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return PreparedCall(lib().pkv_paged_attn_decode_append,
                        common + (_p(out), _p(lse_out), _p(workspace), ws_len, _stream()),
                        (desc, opts, q, k_cache, v_cache, k_new, v_new, block_table,
                         context_lens, out, lse_out, workspace))


def prepare_kv_append_quant(k_cache, v_cache, k_new, v_new, slots, k_scale: float,
                            v_scale: float) -> PreparedCall:
    desc = _check_pools(k_cache, v_cache)
    if k_cache.dtype not in _FP8:
        raise TypeError("kv_append_quant writes fp8 caches")
    _dev(k_new, "k_new")
    _dev(v_new, "v_new", k_new.dtype)
    _dev(slots, "slots", torch.int32)
    n = int(slots.shape[0])
    args = (C.byref(desc), _p(k_cache), _p(v_cache), _p(k_new), _p(v_new),
            _TORCH_TO_CODE[k_new.dtype], float(k_scale), float(v_scale), _p(slots), n, _stream())
    return PreparedCall(lib().pkv_kv_append_quant, args,
                        (desc, k_cache, v_cache, k_new, v_new, slots))


def prepare_merge_states(o_parts, lse_parts, out, lse_out=None) -> PreparedCall:
    _dev(o_parts, "o_parts", torch.float32)
    _dev(lse_parts, "lse_parts", torch.float32)
    _dev(out, "out")
    rows, n, d = (int(x) for x in o_parts.shape)
    args = (_p(o_parts), _p(lse_parts), rows, n, d, _TORCH_TO_CODE[out.dtype], _p(out),
            _p(lse_out), _stream())
    return PreparedCall(lib().pkv_merge_states, args, (o_parts, lse_parts, out, lse_out))


# ---- measurement aids (not the attention path): the ceilings the rooflines
# are read against

def probe_read(buf: torch.Tensor, order: Optional[torch.Tensor] = None, block_bytes: int = 0,
               grid: int = 8192, sink: Optional[torch.Tensor] = None) -> None:
    """pkv_probe_read over the bytes of buf: sequential, or whole blocks of
    block_bytes in the order of `order` (int32 device tensor)."""
    _dev(buf, "buf")
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    if order is not None:
        _dev(order, "order", torch.int32)
    _check(lib().pkv_probe_read(_p(buf), nbytes, _p(order), int(block_bytes), int(grid),
                                _p(sink), _stream()))


def probe_mfma(operands: torch.Tensor, iters: int, vector_work: bool, grid: int,
               clocks: torch.Tensor, sink: Optional[torch.Tensor] = None) -> None:
    """pkv_probe_mfma: operands 4 KiB of bf16 on the device, clocks int64 [2]."""
    _dev(operands, "operands")
    _dev(clocks, "clocks", torch.int64)
    if operands.numel() * operands.element_size() < 4096:
        raise ValueError("operands must hold 256 16-byte vectors")
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=operands.device)
    _check(lib().pkv_probe_mfma(_p(operands), int(iters), 1 if vector_work else 0, int(grid),
                                _p(sink), _p(clocks), _stream()))


def probe_prefill_loop(operands: torch.Tensor, iters: int, vector_work: bool, grid: int,
                       clocks: torch.Tensor, sink: Optional[torch.Tensor] = None) -> None:
    """pkv_probe_prefill_loop: operands 4 KiB of bf16 on the device, clocks int64 [2]."""
    _dev(operands, "operands")
    _dev(clocks, "clocks", torch.int64)
    if operands.numel() * operands.element_size() < 4096:
        raise ValueError("operands must hold 256 16-byte vectors")
    if sink is None:
        sink = torch.zeros(4, dtype=torch.int32, device=operands.device)
    _check(lib().pkv_probe_prefill_loop(_p(operands), int(iters), 1 if vector_work else 0,
                                        int(grid), _p(sink), _p(clocks), _stream()))
