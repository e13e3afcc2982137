"""Seeded synthetic inputs for paged-KV attention.

This module builds page pools, block tables, lengths, slot mappings and
query/key/value tensors.  It holds none of the attention arithmetic: both the
HIP path and the CPU oracle consume what it returns, and neither is imported
here.

The page-pool picture follows the pages' description of a paged KV cache
(page 2, "PageAttention" section 3.2; page 3, section 2.2 "Paged KV Cache"):
fixed-size physical pages taken from a free list, a per-sequence table mapping
logical page i (tokens [i*P, (i+1)*P)) to a physical page id, and physical
pages that need not be contiguous or in order.  Shared prompt prefixes reuse
the same physical pages (page 2, section 3.2, point 2).

Layout (one layer):
  k_cache, v_cache  [num_pages][H_kv][P][D]   cache dtype
  block_table       int32 [B][stride]
  context_lens      int32 [B]
  q                 [B][H_q][D]                (decode)  or  [sum C_b][H_q][D] (prefill)
  k_new, v_new      [n][H_kv][D]               tokens to append
  slots             int32 [n]                  slot = page * P + offset

Poisoning: every pool slot that no sequence covers holds NaN, and table
entries past a sequence's last page point at a page that is all NaN, so a
kernel that reads outside the valid range turns its output into NaN.

Every tensor is drawn from one CPU ``torch.Generator`` per workload, in a
fixed order: lengths, page permutation, Q, K, V, new-token K/V.  Normal draws
are float32 N(0, 1), rounded to the cache dtype (round-to-nearest-even).

fp8 caches (OCP e4m3 / e5m2, one fp32 scale per pool): the stored values are
float32 N(0, 1) draws divided by the pool's scale and converted by torch's own
float8 conversion, so that scale times the stored value follows N(0, 1) up to
the format's rounding.  Q and the new tokens' K/V stay in the query dtype.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

PAGE_SIZE = 16

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "fp8_e4m3": torch.float8_e4m3fn, "fp8_e5m2": torch.float8_e5m2}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3,
               "fp8_e5m2": 4}  # matches pkv_dtype in include/pkv.h
FP8 = ("fp8_e4m3", "fp8_e5m2")

# The five workloads.  Shapes follow the pages' models: Llama-3-8B has 32 query
# heads over 8 KV heads and Llama-3-70B 64 over 8 (page 4, section 2.2 on GQA);
# head_dim 128 and 128K context (page 4, section 2.1 memory table; page 1
# chapter 1 at 128K with batch 8 and tensor parallel 4, so one GPU holds a
# quarter of the heads: 16 query / 2 KV).
CONFIGS: Dict[str, dict] = {
    "tiny": dict(kind="decode", seed=1, batch=4, hq=8, hkv=8, d=64, dtype="f32",
                 lens=[37, 128, 200, 511], num_pages=128, append=False),
    "llama8b": dict(kind="decode", seed=2, batch=64, hq=32, hkv=8, d=128, dtype="bf16",
                    len_range=(512, 4096), pool_slack=0.10, append=True),
    "llama70b_128k": dict(kind="decode", seed=3, batch=8, hq=16, hkv=2, d=128, dtype="f16",
                          ctx=131072, append=True),
    "prefix": dict(kind="decode", seed=4, batch=256, hq=32, hkv=8, d=128, dtype="bf16",
                   prefix=2048, suffix_range=(32, 512), append=False),
    "prefill": dict(kind="prefill", seed=5, batch=4, hq=32, hkv=8, d=128, dtype="bf16",
                    hist=32768, chunk=512),
    # a chunked-prefill batch under page 1's token budget (section 4.1: at most
    # 8192 batched tokens, up to 8 sequences at 128K): 6 sequences decoding one
    # token each at contexts 8K..128K, then 2 prompts each contributing a
    # 4093-row chunk (one at the start of its prompt, one after 64K tokens)
    "mixed": dict(kind="mixed", seed=7, hq=16, hkv=2, d=128, dtype="f16", n_decode=6,
                  decode_range=(8192, 131071), chunk_hist=[0, 65536], chunk=[4093, 4093]),
    # the 128K decode with an fp8 (e4m3) cache: page 1, section 4.1 recommends
    # that cache type for this deployment; f16 queries and outputs
    "llama70b_128k_fp8": dict(kind="decode", seed=6, batch=8, hq=16, hkv=2, d=128,
                              dtype="f16", kv_dtype="fp8_e4m3", k_scale=0.0234375,
                              v_scale=0.01953125, ctx=131072, append=True),
    # the prefill shape over fp8 e5m2 pools (page 4, section 3.1 serves with
    # --kv-cache-dtype fp8_e5m2 and chunked prefill), bf16 queries
    "prefill_fp8": dict(kind="prefill", seed=8, batch=4, hq=32, hkv=8, d=128, dtype="bf16",
                        hist=32768, chunk=512, kv_dtype="fp8_e5m2", k_scale=0.0234375,
                        v_scale=0.01953125),
}


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                      # "decode", "prefill" or "mixed" (decode-first ragged batch)
    dtype: str                     # "f32" | "f16" | "bf16": queries, outputs, new tokens
    num_pages: int
    page_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    batch: int
    k_cache: torch.Tensor          # [num_pages][H_kv][P][D]
    v_cache: torch.Tensor
    q: torch.Tensor                # decode [B][H_q][D]; prefill [sum C][H_q][D]
    block_table: torch.Tensor      # int32 [B][stride]
    context_lens: torch.Tensor     # int32 [B]; decode: tokens attended (after append);
                                   # prefill: history + chunk
    scale: float                   # a float32 value
    k_new: Optional[torch.Tensor] = None   # [n][H_kv][D]
    v_new: Optional[torch.Tensor] = None
    slots: Optional[torch.Tensor] = None   # int32 [n]
    q_indptr: Optional[torch.Tensor] = None  # int32 [B+1] (prefill)
    poison_page: int = -1
    meta: dict = dataclasses.field(default_factory=dict)
    kv_dtype: str = ""             # cache element type ("" = dtype)
    k_scale: float = 1.0           # fp8 caches: K element = k_scale * stored value
    v_scale: float = 1.0

    def __post_init__(self):
        if not self.kv_dtype:
            self.kv_dtype = self.dtype

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODES[self.dtype]

    @property
    def is_fp8(self) -> bool:
        return self.kv_dtype in FP8

    @property
    def stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.batch else 0


def pages_for(n_tokens: int, page_size: int = PAGE_SIZE) -> int:
    """Number of pages a sequence of n_tokens occupies: ceil(n / P)
    (page 1, section 2.3, page-table management)."""
    return (n_tokens + page_size - 1) // page_size


def float32_scale(head_dim: int) -> float:
    """1/sqrt(d) rounded to float32 (the value both sides receive)."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32).item())


def _normal(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(DTYPES[dtype])


def _normal_kv(gen: torch.Generator, shape, kv_dtype: str, scale: float) -> torch.Tensor:
    """Cache contents: N(0, 1) in the cache dtype, or for fp8 N(0, 1) / scale
    converted by torch's float8 conversion."""
    if kv_dtype in FP8:
        x = torch.randn(*shape, generator=gen, dtype=torch.float32)
        x.div_(torch.tensor(scale, dtype=torch.float32))
        return x.to(DTYPES[kv_dtype])
    return _normal(gen, shape, kv_dtype)


def _poison(cache: torch.Tensor, valid: torch.Tensor) -> None:
    """Fill every (page, slot) row not marked valid with NaN, all heads (for
    fp8 the byte 0x7F, a NaN in both OCP formats)."""
    if cache.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        view = cache.view(torch.uint8).permute(0, 2, 1, 3)
        view[~valid] = 0x7F
        return
    view = cache.permute(0, 2, 1, 3)          # [pages][P][H_kv][D] view of the same storage
    view[~valid] = float("nan")


def _build_tables(page_lists: List[List[int]], stride: int, poison_page: int) -> torch.Tensor:
    bt = torch.full((len(page_lists), stride), poison_page, dtype=torch.int32)
    for b, pl in enumerate(page_lists):
        if pl:
            bt[b, : len(pl)] = torch.tensor(pl, dtype=torch.int32)
    return bt


def _valid_mask(num_pages: int, page_lists: List[List[int]], filled: List[int],
                page_size: int) -> torch.Tensor:
    """valid[page][slot] is True where some sequence has a stored token."""
    valid = torch.zeros(num_pages, page_size, dtype=torch.bool)
    for pl, n in zip(page_lists, filled):
        for i, pg in enumerate(pl):
            lo = i * page_size
            cnt = max(0, min(page_size, n - lo))
            if cnt:
                valid[pg, :cnt] = True
    return valid


def _slot_of(page_list: List[int], pos: int, page_size: int) -> int:
    return page_list[pos // page_size] * page_size + pos % page_size


def make_decode(name: str, *, seed: int, batch: int, hq: int, hkv: int, d: int, dtype: str,
                hist_lens: List[int], append: bool, num_pages: Optional[int] = None,
                pool_slack: float = 0.0, shared_prefix: int = 0,
                page_size: int = PAGE_SIZE, gen: Optional[torch.Generator] = None,
                kv_dtype: Optional[str] = None, k_scale: float = 1.0,
                v_scale: float = 1.0) -> Workload:
    """Decode workload.

    hist_lens[b] tokens are already stored.  With ``append`` one more token per
    sequence is handed over as k_new/v_new with its slot; the decode then
    attends to hist_lens[b] + 1 tokens (the appended token included).
    ``shared_prefix`` > 0 makes the first shared_prefix tokens of every
    sequence live in the same physical pages (must be a multiple of P);
    hist_lens then count prefix + suffix.  ``kv_dtype`` (default: dtype) sets
    the cache type; fp8 pools carry k_scale / v_scale and the appended token
    arrives in dtype, to be quantized into the cache.
    """
    kv_dtype = kv_dtype or dtype
    if kv_dtype not in FP8:
        assert kv_dtype == dtype and k_scale == 1.0 and v_scale == 1.0
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    assert shared_prefix % page_size == 0
    ctx = [h + (1 if append else 0) for h in hist_lens]
    pre_pages = shared_prefix // page_size
    own_pages = [pages_for(c, page_size) - pre_pages for c in ctx]
    needed = pre_pages + sum(own_pages)
    if num_pages is None:
        num_pages = int(math.ceil(needed * (1.0 + pool_slack)))
        if num_pages == needed:
            num_pages += 1                      # room for the poison page
    assert num_pages >= needed, "pool too small"
    perm = torch.randperm(num_pages, generator=gen).tolist()
    free = list(perm)                         # free list, popped from the front
    prefix_pages = [free.pop(0) for _ in range(pre_pages)]
    page_lists = []
    for b in range(batch):
        page_lists.append(prefix_pages + [free.pop(0) for _ in range(own_pages[b])])
    poison_page = free[0] if free else -1
    stride = max(len(pl) for pl in page_lists) if page_lists else 1
    stride = max(stride, 1)
    block_table = _build_tables(page_lists, stride, poison_page if poison_page >= 0 else 0)

    q = _normal(gen, (batch, hq, d), dtype)
    k_cache = _normal_kv(gen, (num_pages, hkv, page_size, d), kv_dtype, k_scale)
    v_cache = _normal_kv(gen, (num_pages, hkv, page_size, d), kv_dtype, v_scale)
    valid = _valid_mask(num_pages, page_lists, hist_lens, page_size)
    _poison(k_cache, valid)
    _poison(v_cache, valid)

    k_new = v_new = slots = None
    if append:
        k_new = _normal(gen, (batch, hkv, d), dtype)
        v_new = _normal(gen, (batch, hkv, d), dtype)
        slots = torch.tensor([_slot_of(page_lists[b], hist_lens[b], page_size)
                              for b in range(batch)], dtype=torch.int32)
    return Workload(name=name, kind="decode", dtype=dtype, num_pages=num_pages,
                    page_size=page_size, num_kv_heads=hkv, num_q_heads=hq, head_dim=d,
                    batch=batch, k_cache=k_cache, v_cache=v_cache, q=q,
                    block_table=block_table,
                    context_lens=torch.tensor(ctx, dtype=torch.int32),
                    scale=float32_scale(d), k_new=k_new, v_new=v_new, slots=slots,
                    poison_page=poison_page,
                    meta=dict(page_lists=page_lists, hist_lens=list(hist_lens),
                              shared_prefix=shared_prefix, seed=seed),
                    kv_dtype=kv_dtype, k_scale=float(k_scale), v_scale=float(v_scale))


def make_prefill(name: str, *, seed: int, batch: int, hq: int, hkv: int, d: int, dtype: str,
                 hist: List[int], chunk: List[int], pool_slack: float = 0.0,
                 page_size: int = PAGE_SIZE, gen: Optional[torch.Generator] = None,
                 kv_dtype: Optional[str] = None, k_scale: float = 1.0,
                 v_scale: float = 1.0) -> Workload:
    """Chunked-prefill workload (page 4, section 3.1: the prompt is processed
    in chunks that reuse the KV cache).  hist[b] tokens are stored; chunk[b]
    new query rows follow.  The chunk's own K/V are handed over as k_new/v_new
    with slots at positions hist[b] .. hist[b]+chunk[b]-1; the caller appends
    them before the prefill call, which then attends to hist + chunk tokens.
    ``kv_dtype`` (default: dtype) sets the cache type; fp8 pools carry
    k_scale / v_scale and the chunk's K/V arrive in dtype, to be quantized
    into the cache.
    """
    kv_dtype = kv_dtype or dtype
    if kv_dtype not in FP8:
        assert kv_dtype == dtype and k_scale == 1.0 and v_scale == 1.0
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    total = [h + c for h, c in zip(hist, chunk)]
    own_pages = [pages_for(t, page_size) for t in total]
    needed = sum(own_pages)
    num_pages = int(math.ceil(needed * (1.0 + pool_slack)))
    if num_pages == needed:
        num_pages += 1
    perm = torch.randperm(num_pages, generator=gen).tolist()
    free = list(perm)
    page_lists = [[free.pop(0) for _ in range(n)] for n in own_pages]
    poison_page = free[0]
    stride = max(max(len(pl) for pl in page_lists), 1)
    block_table = _build_tables(page_lists, stride, poison_page)

    n_q = sum(chunk)
    q = _normal(gen, (n_q, hq, d), dtype)
    k_cache = _normal_kv(gen, (num_pages, hkv, page_size, d), kv_dtype, k_scale)
    v_cache = _normal_kv(gen, (num_pages, hkv, page_size, d), kv_dtype, v_scale)
    valid = _valid_mask(num_pages, page_lists, hist, page_size)
    _poison(k_cache, valid)
    _poison(v_cache, valid)
    k_new = _normal(gen, (n_q, hkv, d), dtype)
    v_new = _normal(gen, (n_q, hkv, d), dtype)
    slots = []
    for b in range(batch):
        for i in range(chunk[b]):
            slots.append(_slot_of(page_lists[b], hist[b] + i, page_size))
    indptr = [0]
    for c in chunk:
        indptr.append(indptr[-1] + c)
    return Workload(name=name, kind="prefill", dtype=dtype, num_pages=num_pages,
                    page_size=page_size, num_kv_heads=hkv, num_q_heads=hq, head_dim=d,
                    batch=batch, k_cache=k_cache, v_cache=v_cache, q=q,
                    block_table=block_table,
                    context_lens=torch.tensor(total, dtype=torch.int32),
                    scale=float32_scale(d), k_new=k_new, v_new=v_new,
                    slots=torch.tensor(slots, dtype=torch.int32),
                    q_indptr=torch.tensor(indptr, dtype=torch.int32),
                    poison_page=poison_page,
                    meta=dict(page_lists=page_lists, hist_lens=list(hist),
                              chunk_lens=list(chunk), seed=seed),
                    kv_dtype=kv_dtype, k_scale=float(k_scale), v_scale=float(v_scale))


def make_mixed(name: str, *, seed: int, hq: int, hkv: int, d: int, dtype: str,
               decode_hist: List[int], chunk_hist: List[int], chunk: List[int],
               pool_slack: float = 0.0, gen: Optional[torch.Generator] = None,
               kv_dtype: Optional[str] = None, k_scale: float = 1.0,
               v_scale: float = 1.0) -> Workload:
    """A decode-first ragged batch: len(decode_hist) sequences with one new
    token each (a chunk of one row), then the prompt chunks.  Same layout as a
    prefill workload (every new row's K/V handed over for the append); meta
    carries num_decode."""
    w = make_prefill(name, seed=seed, batch=len(decode_hist) + len(chunk), hq=hq, hkv=hkv, d=d,
                     dtype=dtype, hist=list(decode_hist) + list(chunk_hist),
                     chunk=[1] * len(decode_hist) + list(chunk), pool_slack=pool_slack,
                     gen=gen, kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale)
    w.kind = "mixed"
    w.meta["num_decode"] = len(decode_hist)
    return w


def make(name: str, seed: Optional[int] = None) -> Workload:
    """Build one of the named workloads with its fixed seed (or ``seed``)."""
    cfg = dict(CONFIGS[name])
    seed = cfg.pop("seed") if seed is None else seed
    cfg.pop("seed", None)
    kind = cfg.pop("kind")
    gen = torch.Generator().manual_seed(seed)
    if kind == "mixed":
        lo, hi = cfg["decode_range"]
        dec = torch.randint(lo, hi + 1, (cfg["n_decode"],), generator=gen).tolist()
        return make_mixed(name, seed=seed, hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                          dtype=cfg["dtype"], decode_hist=dec, chunk_hist=cfg["chunk_hist"],
                          chunk=cfg["chunk"], gen=gen)
    if kind == "prefill":
        b = cfg["batch"]
        return make_prefill(name, seed=seed, batch=b, hq=cfg["hq"], hkv=cfg["hkv"],
                            d=cfg["d"], dtype=cfg["dtype"], hist=[cfg["hist"]] * b,
                            chunk=[cfg["chunk"]] * b, gen=gen, kv_dtype=cfg.get("kv_dtype"),
                            k_scale=cfg.get("k_scale", 1.0), v_scale=cfg.get("v_scale", 1.0))
    b = cfg["batch"]
    if name == "tiny":
        hist = list(cfg["lens"])
        return make_decode(name, seed=seed, batch=b, hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                           dtype=cfg["dtype"], hist_lens=hist, append=False,
                           num_pages=cfg["num_pages"], gen=gen)
    if name == "llama8b":
        lo, hi = cfg["len_range"]
        hist = torch.randint(lo, hi + 1, (b,), generator=gen).tolist()
        return make_decode(name, seed=seed, batch=b, hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                           dtype=cfg["dtype"], hist_lens=hist, append=True,
                           pool_slack=cfg["pool_slack"], gen=gen)
    if name in ("llama70b_128k", "llama70b_128k_fp8"):
        hist = [cfg["ctx"] - 1] * b        # the appended token makes the context 131072
        return make_decode(name, seed=seed, batch=b, hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                           dtype=cfg["dtype"], hist_lens=hist, append=True, gen=gen,
                           kv_dtype=cfg.get("kv_dtype"), k_scale=cfg.get("k_scale", 1.0),
                           v_scale=cfg.get("v_scale", 1.0))
    if name == "prefix":
        lo, hi = cfg["suffix_range"]
        suf = torch.randint(lo, hi + 1, (b,), generator=gen).tolist()
        hist = [cfg["prefix"] + s for s in suf]
        return make_decode(name, seed=seed, batch=b, hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                           dtype=cfg["dtype"], hist_lens=hist, append=False,
                           shared_prefix=cfg["prefix"], gen=gen)
    raise KeyError(name)


def duplicate_shared_pages(w: Workload) -> Workload:
    """Copy of a shared-prefix workload in which every sequence owns a private
    copy of the prefix pages (same bytes, distinct physical pages)."""
    pre = w.meta.get("shared_prefix", 0) // w.page_size
    assert pre > 0
    pl = w.meta["page_lists"]
    shared = pl[0][:pre]
    extra = pre * (w.batch - 1)
    n_pages = w.num_pages + extra
    k = torch.empty((n_pages,) + tuple(w.k_cache.shape[1:]), dtype=w.k_cache.dtype)
    v = torch.empty_like(k)
    k[: w.num_pages] = w.k_cache
    v[: w.num_pages] = w.v_cache
    new_lists = [list(pl[0])]
    nxt = w.num_pages
    for b in range(1, w.batch):
        own = []
        for pg in shared:
            k[nxt] = w.k_cache[pg]
            v[nxt] = w.v_cache[pg]
            own.append(nxt)
            nxt += 1
        new_lists.append(own + list(pl[b][pre:]))
    bt = _build_tables(new_lists, w.stride, w.poison_page)
    out = dataclasses.replace(w, num_pages=n_pages, k_cache=k, v_cache=v, block_table=bt,
                              meta=dict(w.meta, page_lists=new_lists, shared_prefix=0))
    return out


def permute_pages(w: Workload, seed: int) -> Workload:
    """Same logical cache with the physical pages renumbered by a random
    permutation pi: new page pi[p] holds old page p, tables are remapped."""
    gen = torch.Generator().manual_seed(seed)
    pi = torch.randperm(w.num_pages, generator=gen)
    k = torch.empty_like(w.k_cache)
    v = torch.empty_like(w.v_cache)
    k[pi] = w.k_cache
    v[pi] = w.v_cache
    bt = pi[w.block_table.long()].to(torch.int32)
    slots = None
    if w.slots is not None:
        s = w.slots.long()
        pg = pi[s // w.page_size]
        slots = (pg * w.page_size + s % w.page_size).to(torch.int32)
    lists = [[int(pi[p]) for p in pl] for pl in w.meta.get("page_lists", [])]
    return dataclasses.replace(w, k_cache=k, v_cache=v, block_table=bt, slots=slots,
                               poison_page=int(pi[w.poison_page]) if w.poison_page >= 0 else -1,
                               meta=dict(w.meta, page_lists=lists))


def contiguous_kv(w: Workload, b: int):
    """Logical K/V rows of sequence b as contiguous tensors [L][H_kv][D]
    (after any append has been applied to w's pools by the caller)."""
    n = int(w.context_lens[b])
    pl = w.meta["page_lists"][b]
    ks, vs = [], []
    for i in range(pages_for(n, w.page_size)):
        cnt = min(w.page_size, n - i * w.page_size)
        ks.append(w.k_cache[pl[i], :, :cnt, :].permute(1, 0, 2))
        vs.append(w.v_cache[pl[i], :, :cnt, :].permute(1, 0, 2))
    if not ks:
        shape = (0, w.num_kv_heads, w.head_dim)
        return torch.empty(shape, dtype=w.k_cache.dtype), torch.empty(shape, dtype=w.v_cache.dtype)
    return torch.cat(ks, 0).contiguous(), torch.cat(vs, 0).contiguous()

