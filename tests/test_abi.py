"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and every invalid-argument path returns its status before
any HIP call (fake, aligned device addresses are never dereferenced)."""
import ctypes as C
import math

import pytest
import torch

from paged_kv_cache_04_amd import binding
from paged_kv_cache_04_amd.binding import CacheDesc


@pytest.fixture(scope="module")
def L():
    return binding.lib()


FAKE = C.c_void_p(1 << 20)        # aligned, never dereferenced on these paths


def desc(num_pages=64, page_size=16, hkv=2, d=128, dtype=2):
    return CacheDesc(num_pages, page_size, hkv, d, dtype)


def test_exports_every_declared_symbol(L):
    names = binding.declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert L.pkv_version() == 4


def err(L):
    return L.pkv_last_error().decode()


def test_desc_checks(L):
    assert L.pkv_kv_append(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == -1
    for d, code, words in [(desc(page_size=32), -2, "page_size"), (desc(d=96), -2, "head_dim"),
                           (desc(dtype=7), -1, "dtype"), (desc(num_pages=0), -1, "num_pages"),
                           (desc(hkv=0), -1, "num_kv_heads"), (desc(page_size=0), -1, "page_size")]:
        rc = L.pkv_kv_append(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 1, None)
        assert rc == code and words in err(L)


def test_append_args(L):
    d = desc()
    assert L.pkv_kv_append(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, -1, None) == -1
    assert L.pkv_kv_append(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == 0
    assert L.pkv_kv_append(C.byref(d), FAKE, None, FAKE, FAKE, FAKE, 4, None) == -1
    assert L.pkv_kv_append(C.byref(d), C.c_void_p((1 << 20) + 4), FAKE, FAKE, FAKE, FAKE, 4,
                           None) == -1
    assert "aligned" in err(L)


def _decode(L, d, *, batch=2, hq=4, stride=8, max_len=100, split=0, ws=None, ws_bytes=0,
            out=FAKE, q=FAKE):
    return L.pkv_paged_attn_decode(C.byref(d), FAKE, FAKE, q, batch, hq, FAKE, stride, FAKE,
                                   max_len, 0.125, split, out, None, ws, ws_bytes, None)


def test_decode_args(L):
    d = desc()
    assert _decode(L, d, hq=3) == -1                       # not a multiple of H_kv
    assert _decode(L, d, hq=64) == -2                      # G = 32 not built
    assert _decode(L, desc(d=64), hq=32) == -2             # G = 16: head_dim 128 only
    assert "16 query heads" in err(L)
    assert _decode(L, desc(dtype=0), hq=32) == -2          # G = 16: 16-bit queries only
    assert _decode(L, d, max_len=8 * 16 + 1) == -1         # beyond stride * P
    assert _decode(L, d, batch=-1) == -1
    assert _decode(L, d, split=24) == -1                   # not a multiple of P
    assert _decode(L, d, out=None) == -1
    assert _decode(L, d, q=None) == -1
    assert _decode(L, d, batch=0) == 0                     # empty batch: no-op


def test_decode_workspace_required_when_split(L):
    d = desc()
    n = C.c_int32()
    ws = C.c_size_t()
    assert L.pkv_decode_plan(C.byref(d), 2, 4, 128, 32, C.byref(n), C.byref(ws)) == 0
    assert n.value == 4
    rows = 2 * 4
    o_bytes = (rows * 4 * 128 * 4 + 255) // 256 * 256
    assert ws.value == o_bytes + rows * 4 * 4
    assert _decode(L, d, max_len=128, split=32, ws=FAKE, ws_bytes=ws.value - 1) == -3
    assert "workspace" in err(L)
    assert _decode(L, d, max_len=128, split=32, ws=None, ws_bytes=0) == -3


def test_noalloc_args(L):
    """The decode step on the static scratch array: argument checks as the
    workspace form, and a split plan larger than the array is refused before
    any HIP call."""
    assert L.pkv_noalloc_scratch_bytes() == 16 << 20
    d = desc(hkv=8)

    def call(batch=64, hq=32, stride=256, max_len=4096, split=0, q=FAKE, out=FAKE):
        return L.pkv_paged_attn_decode_append_noalloc(
            C.byref(d), FAKE, FAKE, FAKE, FAKE, q, batch, hq, FAKE, stride, FAKE, max_len,
            0.125, split, None, out, None, None)

    # 64 x 32 rows x 256 splits x 129 floats: 270 MB of partials
    assert call(split=16) == -3 and "static scratch" in err(L)
    assert call(batch=0) == 0
    assert call(hq=12) == -1
    assert call(split=24) == -1
    assert call(max_len=256 * 16 + 1) == -1
    assert call(q=None) == -1
    assert call(out=None) == -1


@pytest.mark.parametrize("name,batch,hq,hkv,max_len,want_split", [
    ("llama70b_128k", 8, 16, 2, 131072, 16),       # G 8: matrix-core kernel, 256 workgroups
    ("llama70b_128k, G 4", 8, 8, 2, 131072, 16),   # G 4, 16-bit: matrix cores too, 256
    ("llama70b_128k, G 2", 8, 4, 2, 131072, 32),   # G 2: vector kernel, 512
    ("tiny", 4, 8, 8, 511, 1),                     # at most 32 pages: no split
    ("33 pages", 4, 8, 8, 513, 3),
    ("prefix", 256, 32, 8, 2560, 1),
])
def test_auto_plan(L, name, batch, hq, hkv, max_len, want_split):
    d = desc(hkv=hkv)
    n = C.c_int32()
    ws = C.c_size_t()
    assert L.pkv_decode_plan(C.byref(d), batch, hq, max_len, 0, C.byref(n), C.byref(ws)) == 0
    assert n.value == want_split
    assert (ws.value == 0) == (n.value == 1)


def test_plan_group_16(L):
    """G = 16 plans on the matrix-core decode (head_dim 128, 16-bit queries)."""
    n = C.c_int32()
    ws = C.c_size_t()
    assert L.pkv_decode_plan(C.byref(desc()), 8, 32, 131072, 0, C.byref(n), C.byref(ws)) == 0
    assert n.value == 16
    assert L.pkv_decode_plan(C.byref(desc(dtype=0)), 8, 32, 4096, 0, C.byref(n),
                             C.byref(ws)) == -2


def test_split_for_lens(L):
    """The lengths-aware split: equal lengths give the automatic split; an
    uneven batch spreads its visited pages over ~1024 workgroups of at least
    32 pages; a window counts only the pages it visits."""
    d = desc(num_pages=65537, dtype=1)
    out = C.c_int32()

    def split(lens, hq=16, opts=None):
        arr = (C.c_int32 * len(lens))(*lens)
        rc = L.pkv_decode_split_for_lens(C.byref(d), len(lens), hq, arr,
                                         C.byref(opts) if opts else None, C.byref(out))
        return rc, out.value

    assert split([131072] * 8) == (0, 8192)                 # the automatic 16 splits
    lens = [8192, 40000, 70000, 100000, 131071, 20000]
    rc, s = split(lens)
    assert rc == 0 and s % 16 == 0
    pps = s // 16
    active = 2 * sum(math.ceil(math.ceil(n / 16) / pps) for n in lens)   # x 2 KV heads
    assert 0.95 * 1024 <= active <= 1024 + 2 * len(lens)    # split size rounds up
    opts = binding.DecodeOpts(1, 1.0, 1.0, 4096, 128)
    assert split([131072] * 8, opts=opts) == (0, 272)       # 17 of the window's 265 pages
    # both visit 264 pages: the automatic split of that batch (17 splits of 16 pages)
    n, ws = C.c_int32(), C.c_size_t()
    assert L.pkv_decode_plan_ex(C.byref(d), 2, 16, 131072, 0, C.byref(opts), C.byref(n),
                                C.byref(ws)) == 0
    assert split([131072, 100000], opts=opts) == (0, 16 * math.ceil(265 / n.value))
    assert split([100, 200])[1] == 32 * 16                  # at least 32 pages per split
    assert split([16 * 64, 160]) == (0, 32 * 16)            # never below 32 pages
    assert L.pkv_decode_plan(C.byref(d), 64, 32, 4096, 0, C.byref(n), C.byref(ws)) == 0
    assert split([4096] * 64, hq=32) == (0, 16 * math.ceil(256 / n.value))   # equal: automatic
    assert split([5, -1])[0] == -1
    assert split([5], hq=5)[0] == -1
    assert L.pkv_decode_split_for_lens(C.byref(d), 1, 16, None, None, C.byref(out)) == -1
    assert L.pkv_decode_split_for_lens(C.byref(desc(dtype=0)), 1, 32,
                                       (C.c_int32 * 1)(5), None, C.byref(out)) == -2


def test_merge_args(L):
    assert L.pkv_merge_states(FAKE, FAKE, -1, 2, 128, 0, FAKE, None, None) == -1
    assert L.pkv_merge_states(FAKE, FAKE, 4, 0, 128, 0, FAKE, None, None) == -1
    assert L.pkv_merge_states(FAKE, FAKE, 4, 2, 128, 9, FAKE, None, None) == -1
    assert L.pkv_merge_states(FAKE, FAKE, 0, 2, 128, 0, FAKE, None, None) == 0


def test_validate_tables():
    d = desc(num_pages=10)
    bt = torch.tensor([[3, 4, 0], [9, 1, 1]], dtype=torch.int32)
    binding.validate_tables(d, bt, torch.tensor([40, 17], dtype=torch.int32),
                            torch.tensor([5, -1, 159], dtype=torch.int32))
    with pytest.raises(binding.PkvError, match="block_table"):
        binding.validate_tables(d, torch.tensor([[3, 10, 0]], dtype=torch.int32),
                                torch.tensor([17], dtype=torch.int32))
    with pytest.raises(binding.PkvError, match="lens"):
        binding.validate_tables(d, bt, torch.tensor([49, 1], dtype=torch.int32))
    with pytest.raises(binding.PkvError, match="repeats"):
        binding.validate_tables(d, bt, torch.tensor([40, 17], dtype=torch.int32),
                                torch.tensor([5, 5], dtype=torch.int32))
    with pytest.raises(binding.PkvError, match="slot"):
        binding.validate_tables(d, bt, torch.tensor([40, 17], dtype=torch.int32),
                                torch.tensor([160], dtype=torch.int32))
    # entries past ceil(len / P) are not checked (they may point anywhere)
    binding.validate_tables(d, torch.tensor([[3, -7, 99]], dtype=torch.int32),
                            torch.tensor([16], dtype=torch.int32))


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        binding.kv_append(x, x, x[0], x[0], torch.zeros(4, dtype=torch.int32))


def _prefill(L, d, *, batch=2, hq=4, total=10, max_q=8, stride=8, max_kv=100, q=FAKE):
    return L.pkv_paged_attn_prefill_chunk(C.byref(d), FAKE, FAKE, q, FAKE, batch, hq, total,
                                          max_q, FAKE, stride, FAKE, max_kv, 0.125, FAKE, None,
                                          None)


def test_prefill_args(L):
    assert _prefill(L, desc(dtype=0)) == -2              # f32 is not built on MFMA
    assert _prefill(L, desc(d=64), batch=0) == 0         # head_dim 64: 16-bit pools
    assert _prefill(L, desc(), hq=3) == -1
    assert _prefill(L, desc(), max_kv=8 * 16 + 1) == -1
    assert _prefill(L, desc(), max_q=200) == -1          # longer than max_kv
    assert _prefill(L, desc(), q=None) == -1
    assert _prefill(L, desc(), total=-1) == -1
    assert _prefill(L, desc(), batch=0) == 0


def _opts(q_dtype=2, k_scale=1.0, v_scale=1.0, window=0, sink=0):
    return binding.DecodeOpts(q_dtype, k_scale, v_scale, window, sink)


def _decode_ex(L, d, opts, *, batch=2, hq=4, stride=8, max_len=100, split=0):
    return L.pkv_paged_attn_decode_ex(C.byref(d), FAKE, FAKE, FAKE, batch, hq, FAKE, stride,
                                      FAKE, max_len, 0.125, split,
                                      None if opts is None else C.byref(opts), FAKE, None,
                                      None, 0, None)


def test_decode_ex_options(L):
    f8 = desc(dtype=3)
    assert _decode(L, f8) == -1 and "q_dtype" in err(L)       # fp8 needs options
    assert _decode_ex(L, f8, _opts(q_dtype=0)) == -2          # f32 queries over fp8
    assert _decode_ex(L, f8, _opts(q_dtype=3)) == -2
    assert _decode_ex(L, desc(dtype=3, d=64), _opts(q_dtype=1)) == -2   # fp8 needs D 128
    assert _decode_ex(L, f8, _opts(q_dtype=1, k_scale=0.0)) == -1
    assert _decode_ex(L, f8, _opts(q_dtype=1, v_scale=float("inf"))) == -1
    assert _decode_ex(L, f8, _opts(q_dtype=1, window=-1)) == -1
    assert _decode_ex(L, f8, _opts(q_dtype=2), batch=0) == 0
    bf = desc(dtype=2)
    assert _decode_ex(L, bf, _opts(q_dtype=1)) == -1           # q type must match
    assert _decode_ex(L, bf, _opts(k_scale=2.0)) == -1         # scales are fp8-only
    assert _decode_ex(L, bf, None, batch=0) == 0
    assert _decode_ex(L, bf, _opts(window=4, sink=2), batch=0) == 0


def test_plan_ex_counts_window_pages_only(L):
    d = desc(hkv=2)
    n, ws = C.c_int32(), C.c_size_t()
    assert L.pkv_decode_plan_ex(C.byref(d), 8, 16, 131072, 0, None, C.byref(n), C.byref(ws)) == 0
    assert n.value == 16
    o = _opts(q_dtype=2, window=4096, sink=128)
    assert L.pkv_decode_plan_ex(C.byref(d), 8, 16, 131072, 0, C.byref(o), C.byref(n),
                                C.byref(ws)) == 0
    # (128/16 + 4096/16 + 1) pages = 265 pages -> at most 17 splits of >= 16 pages
    assert 1 <= n.value <= 17
    o = _opts(q_dtype=2, window=4096, sink=128)
    assert L.pkv_decode_plan_ex(C.byref(d), 8, 16, 131072, 1024, C.byref(o), C.byref(n),
                                C.byref(ws)) == 0
    assert n.value == (265 * 16 + 1023) // 1024


def test_kv_append_quant_args(L):
    f8 = desc(dtype=4)
    q = L.pkv_kv_append_quant
    assert q(C.byref(desc(dtype=2)), FAKE, FAKE, FAKE, FAKE, 2, 1.0, 1.0, FAKE, 4, None) == -1
    assert q(C.byref(f8), FAKE, FAKE, FAKE, FAKE, 3, 1.0, 1.0, FAKE, 4, None) == -2
    assert q(C.byref(f8), FAKE, FAKE, FAKE, FAKE, 9, 1.0, 1.0, FAKE, 4, None) == -1
    assert q(C.byref(f8), FAKE, FAKE, FAKE, FAKE, 2, 0.0, 1.0, FAKE, 4, None) == -1
    assert q(C.byref(f8), FAKE, FAKE, FAKE, FAKE, 2, 1.0, float("nan"), FAKE, 4, None) == -1
    assert q(C.byref(f8), FAKE, FAKE, FAKE, FAKE, 2, 1.0, 1.0, FAKE, -1, None) == -1
    assert q(C.byref(f8), FAKE, FAKE, FAKE, FAKE, 2, 1.0, 1.0, FAKE, 0, None) == 0


def test_fp8_elsewhere_rejected(L):
    assert _prefill(L, desc(dtype=3)) == -1      # fp8 pools need the _ex form's query type
    assert L.pkv_merge_states(FAKE, FAKE, 4, 2, 128, 3, FAKE, None, None) == -2


def _prefill_ex(L, d, opts, *, batch=2, hq=4, total=10, max_q=8, stride=8, max_kv=100):
    return L.pkv_paged_attn_prefill_chunk_ex(C.byref(d), FAKE, FAKE, FAKE, FAKE, batch, hq, total,
                                             max_q, FAKE, stride, FAKE, max_kv, 0.125,
                                             None if opts is None else C.byref(opts), FAKE, None,
                                             None)


def _mixed_ex(L, d, opts, *, batch=4, nd=2, total=10, max_q=8, stride=8, max_kv=100):
    return L.pkv_paged_attn_mixed_ex(C.byref(d), FAKE, FAKE, FAKE, FAKE, batch, nd, 4, total,
                                     max_q, FAKE, stride, FAKE, max_kv, 0.125, 0,
                                     None if opts is None else C.byref(opts), FAKE, None, None, 0,
                                     None)


def test_prefill_and_mixed_ex_args(L):
    f8, f16 = desc(dtype=3), desc(dtype=1)
    ok = _opts(1, 0.5, 0.25)
    # host checks pass; nothing to launch with no sequences or no rows
    assert _prefill_ex(L, f8, ok, batch=0) == 0
    assert _prefill_ex(L, desc(dtype=4), _opts(2, 0.5, 0.25), total=0) == 0
    assert _mixed_ex(L, f8, ok, batch=0, nd=0) == 0
    assert _prefill_ex(L, f16, None, batch=0) == 0            # NULL options: the plain call
    assert _prefill_ex(L, f8, None, batch=0) == -1            # fp8 needs a query type
    assert _prefill_ex(L, f8, _opts(3), batch=0) == -2        # fp8 queries are not built
    assert _prefill_ex(L, f8, _opts(1, 0.0, 1.0), batch=0) == -1      # scales > 0
    assert _prefill_ex(L, f8, _opts(1, 1.0, float("inf")), batch=0) == -1
    assert _prefill_ex(L, f16, _opts(2), batch=0) == -1       # 16-bit pools: q_dtype = dtype
    assert _prefill_ex(L, f16, _opts(1, 2.0, 1.0), batch=0) == -1     # scales: fp8 only
    assert _prefill_ex(L, f8, _opts(1, 1.0, 1.0, 64, 0), batch=0) == -1   # no window here
    assert _prefill_ex(L, f8, _opts(1, 1.0, 1.0, 0, 4), batch=0) == -1    # nor a sink
    assert _mixed_ex(L, f8, _opts(1, 1.0, 1.0, 64, 0), batch=0, nd=0) == -1
    assert _prefill_ex(L, desc(dtype=3, d=64), ok, batch=0) == -2     # head_dim 128 only
    assert _prefill_ex(L, desc(dtype=0), _opts(0), batch=0) == -2     # f32: not on MFMA
    assert _mixed_ex(L, f8, ok, nd=5) == -1                   # more decode rows than sequences


def _mixed(L, d, *, batch=4, nd=2, total=10, max_q=8, stride=8, max_kv=100):
    return L.pkv_paged_attn_mixed(C.byref(d), FAKE, FAKE, FAKE, FAKE, batch, nd, 4, total, max_q,
                                  FAKE, stride, FAKE, max_kv, 0.125, 0, FAKE, None, None, 0,
                                  None)


def test_mixed_args(L):
    d = desc()
    assert _mixed(L, d, nd=-1) == -1
    assert _mixed(L, d, nd=5) == -1                       # more decode rows than sequences
    assert _mixed(L, d, nd=3, total=2) == -1              # more decode rows than q rows
    assert _mixed(L, d, nd=1, max_q=0) == -1              # chunks need max_q_len >= 1
    assert _mixed(L, desc(dtype=0)) == -2                 # the chunk path is MFMA: f16/bf16
    assert _mixed(L, d, batch=0, nd=0) == 0


def _shared(L, d, opts=None, *, batch=2, hq=4, prefix=256, stride=8, max_suffix=100,
            ws=FAKE, ws_bytes=1 << 30, prefix_table=FAKE, out=FAKE):
    return L.pkv_paged_attn_decode_shared_prefix(
        C.byref(d), FAKE, FAKE, FAKE, batch, hq, prefix_table, prefix, FAKE, stride, FAKE,
        max_suffix, 0.125, 0, None if opts is None else C.byref(opts), out, None, ws, ws_bytes,
        None)


def test_shared_prefix_plan_and_args(L):
    d = desc(num_pages=10000, hkv=8)
    n, ws = C.c_int32(), C.c_size_t()

    def plan(batch, hq, prefix, max_suffix, split=0, dd=d, opts=None):
        rc = L.pkv_decode_shared_prefix_plan(C.byref(dd), batch, hq, prefix, max_suffix, split,
                                             None if opts is None else C.byref(opts),
                                             C.byref(n), C.byref(ws))
        return rc, n.value, ws.value

    # the 256-sequence batch sharing 2048 tokens: 8 splits of the shared keys
    # (8 KV heads x 4 row tiles x 8 = 256 workgroups) + the own pages' split
    rc, parts, wsb = plan(256, 32, 2048, 513)
    assert rc == 0 and parts == 9
    rows = 256 * 32
    assert wsb == (rows * parts * 128 * 4 + 255) // 256 * 256 + rows * parts * 4
    rc, parts, _ = plan(6, 16, 0, 701)            # no shared pages: the decode's own splits
    m = C.c_int32()
    assert L.pkv_decode_plan(C.byref(d), 6, 16, 701, 0, C.byref(m), C.byref(ws)) == 0
    assert rc == 0 and parts == m.value
    assert plan(2, 16, 100, 10)[0] == -1          # shared part not whole pages
    assert plan(2, 16, -16, 10)[0] == -1
    assert plan(2, 16, 256, -1)[0] == -1
    assert plan(2, 16, 256, 10, dd=desc(dtype=0))[0] == -2       # f32 pools
    assert plan(2, 16, 256, 10, dd=desc(d=64))[0] == 0           # head_dim 64, 16-bit
    assert plan(2, 16, 256, 10, dd=desc(d=64, dtype=3), opts=_opts(1))[0] == -2   # fp8: 128
    assert plan(2, 16, 256, 10, opts=_opts(2, 1.0, 1.0, 64, 0))[0] == -1   # no window
    # the call: host checks before any launch
    assert _shared(L, desc(), prefix=100) == -1
    assert _shared(L, desc(), prefix_table=None) == -1
    assert _shared(L, desc(), out=None) == -1
    assert _shared(L, desc(), ws=None) == -3
    assert _shared(L, desc(), ws_bytes=16) == -3
    assert _shared(L, desc(), max_suffix=8 * 16 + 1) == -1     # beyond stride * P
    assert _shared(L, desc(), batch=0) == 0
    assert _shared(L, desc(dtype=3), batch=0) == -1             # fp8: needs the query type
    assert _shared(L, desc(dtype=3), _opts(1, 0.5, 0.5), batch=0) == 0


def _decode_append(L, d, opts=None, *, partials=False, batch=2, hq=4, stride=8, max_len=100,
                   split=0, k_new=FAKE, v_new=FAKE, ws=None, ws_bytes=0, out=FAKE):
    lead = (C.byref(d), FAKE, FAKE, k_new, v_new, FAKE, batch, hq, FAKE, stride, FAKE, max_len,
            0.125, split, C.byref(opts) if opts is not None else None)
    if partials:
        return L.pkv_paged_attn_decode_append_partials(*lead, ws, ws_bytes, None)
    return L.pkv_paged_attn_decode_append(*lead, out, None, ws, ws_bytes, None)


def test_decode_append_args(L):
    """The decode-with-append calls check what the decode calls check, plus
    the new rows: both present and 16-byte aligned (an empty batch needs
    neither)."""
    d = desc()
    for partials in (False, True):
        kw = dict(partials=partials)
        assert _decode_append(L, d, k_new=None, **kw) == -1
        assert "k_new" in err(L)
        assert _decode_append(L, d, v_new=None, **kw) == -1
        assert _decode_append(L, d, k_new=C.c_void_p((1 << 20) + 2), **kw) == -1
        assert "aligned" in err(L)
        assert _decode_append(L, d, hq=3, **kw) == -1                 # not a multiple of H_kv
        assert _decode_append(L, d, max_len=8 * 16 + 1, **kw) == -1   # beyond stride * P
        assert _decode_append(L, d, batch=0, k_new=None, v_new=None, **kw) == 0
        f8 = desc(dtype=3)
        assert _decode_append(L, f8, **kw) == -1                      # fp8 needs a q type
        assert _decode_append(L, f8, _opts(q_dtype=1, k_scale=0.0), **kw) == -1
        assert _decode_append(L, f8, _opts(q_dtype=1), batch=0, **kw) == 0
    # the full call needs out, and a workspace once split; the partials need a workspace
    assert _decode_append(L, d, out=None) == -1
    assert _decode_append(L, d, max_len=128, split=32) == -3
    assert _decode_append(L, d, partials=True) == -3



@pytest.mark.parametrize("name", ["pkv_probe_mfma", "pkv_probe_prefill_loop"])
def test_matrix_probe_args(L, name):
    """The measurement probes reject bad arguments before any HIP call."""
    f = getattr(L, name)
    assert f(None, 10, 0, 1, FAKE, FAKE, None) == -1                     # operands
    assert f(FAKE, 10, 0, 1, None, FAKE, None) == -1                     # sink
    assert f(FAKE, 10, 0, 1, FAKE, None, None) == -1                     # clocks
    assert f(C.c_void_p((1 << 20) + 4), 10, 0, 1, FAKE, FAKE, None) == -1
    assert "aligned" in err(L)
    assert f(FAKE, 0, 0, 1, FAKE, FAKE, None) == -1                      # iters
    assert f(FAKE, 10, 0, 0, FAKE, FAKE, None) == -1                     # grid
    assert f(FAKE, 10, 2, 1, FAKE, FAKE, None) == -1                     # vector_work
    assert "vector_work" in err(L)
