"""GPU parity of kv_append, gather and paged decode against the CPU oracle,
through the C ABI (libpkv.so via the binding)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_04_amd as pkv
from oracle import pkvref
from paged_kv_cache_04_amd import workloads as W

from helpers import assert_close, assert_lse_close, bits, host_threads, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu_decode(w, d, split_tokens=0):
    if w.k_new is not None:
        pkv.kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"])
    out, lse = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                     d["context_lens"], w.max_context_len, w.scale,
                                     split_tokens=split_tokens, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(w, rows=None):
    if w.k_new is not None:
        pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
    return pkvref.decode(w.dtype, w.k_cache, w.v_cache, w.q, w.block_table, w.context_lens,
                         w.scale, rows=rows, n_threads=host_threads())


def check_decode(w, split_tokens=0, what=""):
    d = to_dev(w, DEV)
    out, lse = gpu_decode(w, d, split_tokens)
    ref, ref_lse = oracle_decode(w)
    # the pool after the append is bit-identical to the oracle's
    assert torch.equal(bits(d["k_cache"]), bits(w.k_cache)), "k pool after append"
    assert torch.equal(bits(d["v_cache"]), bits(w.v_cache)), "v pool after append"
    assert_close(out.reshape(ref.shape), ref, w.dtype, what or w.name)
    assert_lse_close(lse.reshape(-1), ref_lse, w.dtype, what or w.name)
    return out, lse


# ----------------------------------------------------------------- configs

@pytest.mark.parametrize("name", ["tiny", "llama8b", "prefix"])
def test_decode_config_parity(name):
    w = W.make(name)
    print(f"[decode parity] {name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"D={w.head_dim} {w.dtype}", flush=True)
    check_decode(w)


def test_decode_llama70b_128k_parity():
    """Full size: 8 x 131072 keys, GQA 8, split-KV + merge, every output row."""
    w = W.make("llama70b_128k")
    print("[decode parity] llama70b_128k full size", flush=True)
    check_decode(w)


@pytest.mark.parametrize("dtype,d,hq,hkv", [
    ("f32", 64, 2, 2), ("f32", 128, 8, 1), ("f32", 64, 8, 1), ("f32", 128, 4, 2),
    ("f32", 128, 8, 2),                      # f32 at head_dim 128, G 4 and 8: a wave per SIMD
    ("f16", 64, 4, 2), ("f16", 128, 2, 1), ("f16", 64, 8, 1), ("f16", 128, 1, 1),
    ("bf16", 64, 16, 2), ("bf16", 128, 6, 3), ("bf16", 64, 1, 1), ("bf16", 128, 16, 16),
    ("bf16", 64, 8, 2),                      # G = 4 at head_dim 64: the vector kernel
    # G = 4, 8 and 16 at head_dim 128: the matrix-core kernel
    ("f16", 128, 16, 2), ("bf16", 128, 8, 1), ("bf16", 128, 32, 4), ("f16", 128, 32, 2),
    ("bf16", 128, 16, 1), ("f16", 128, 8, 2), ("bf16", 128, 4, 1),
])
def test_decode_shapes(dtype, d, hq, hkv):
    """Every (dtype, head_dim, group) kernel variant, ragged lengths spanning
    several pages and splits, last pages partial."""
    lens = [0, 1, 15, 16, 17, 100, 257, 700]
    w = W.make_decode("shape", seed=hq * 7 + d, batch=len(lens), hq=hq, hkv=hkv, d=d,
                      dtype=dtype, hist_lens=[max(0, l - 1) for l in lens], append=True,
                      pool_slack=0.3)
    lens_eff = w.context_lens.tolist()
    assert lens_eff[0] == 1
    for split in (0, 64):
        w2 = W.make_decode("shape", seed=hq * 7 + d, batch=len(lens), hq=hq, hkv=hkv, d=d,
                           dtype=dtype, hist_lens=[max(0, l - 1) for l in lens], append=True,
                           pool_slack=0.3)
        check_decode(w2, split_tokens=split, what=f"{dtype} D{d} G{hq // hkv} split {split}")


def test_empty_context_rows():
    w = W.make_decode("empty", seed=3, batch=3, hq=4, hkv=2, d=128, dtype="bf16",
                      hist_lens=[0, 5, 0], append=False, pool_slack=0.5)
    d = to_dev(w, DEV)
    for split in (0, 16):
        out, lse = gpu_decode(w, d, split)
        assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
        assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[2]))
        assert torch.isfinite(out[1].float()).all()


# --------------------------------------------------------------- indexing

@pytest.mark.parametrize("dtype,group", [("f32", 4), ("f16", 4), ("bf16", 4), ("f16", 8),
                                         ("bf16", 8), ("f16", 16)])
def test_one_hot_key_bit_exact(dtype, group):
    """K = 0 except the target token's key, whose score is >= 200: every other
    weight underflows to exactly 0, so the output is V[target] bit for bit.
    Targets sweep page boundaries and the last token (G = 8, 16: matrix cores)."""
    L = 300
    targets = [0, 15, 16, 17, 31, 32, 150, 255, 256, 298, 299]
    w = W.make_decode("onehot", seed=5, batch=len(targets), hq=2 * group, hkv=2, d=128,
                      dtype=dtype, hist_lens=[L] * len(targets), append=False, pool_slack=0.1)
    k = torch.zeros_like(w.k_cache)
    k[torch.isnan(w.k_cache)] = float("nan")          # keep the poison
    q = torch.zeros_like(w.q)
    q[:, :, 0] = 1.0
    big = 2304.0                                      # exact in f16/bf16; score 2304/sqrt(128) > 200
    for b, t in enumerate(targets):
        pg = w.meta["page_lists"][b][t // 16]
        k[pg, :, t % 16, 0] = big
    w.k_cache, w.q = k, q
    d = to_dev(w, DEV)
    G = group
    for split in (0, 16, 64, 128):
        out, _ = gpu_decode(w, d, split)
        for b, t in enumerate(targets):
            pg = w.meta["page_lists"][b][t // 16]
            for h in range(2 * group):
                want = w.v_cache[pg, h // G, t % 16]
                assert torch.equal(bits(out[b, h]), bits(want)), (dtype, split, t, h)


def test_length_one_bit_exact():
    w = W.make_decode("l1", seed=6, batch=5, hq=8, hkv=1, d=64, dtype="bf16",
                      hist_lens=[1] * 5, append=False)
    d = to_dev(w, DEV)
    out, lse = gpu_decode(w, d)
    for b in range(5):
        pg = w.meta["page_lists"][b][0]
        for h in range(8):
            assert torch.equal(bits(out[b, h]), bits(w.v_cache[pg, 0, 0]))


def test_gather_bit_exact():
    w = W.make("llama8b")
    d = to_dev(w, DEV)
    pkv.kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"])
    pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
    for b in (0, 17, 63):
        L = int(w.context_lens[b])
        kg, vg = pkv.gather_kv(d["k_cache"], d["v_cache"], d["block_table"][b].contiguous(), L)
        kr, vr = pkvref.gather(w.dtype, w.k_cache, w.v_cache, w.block_table[b], L)
        assert torch.equal(bits(kg), bits(kr)) and torch.equal(bits(vg), bits(vr))


def test_kv_append_chunk_bit_exact():
    """Append of a 2048-token prefill chunk (with a skipped slot) over the
    whole pool: touched slots equal the oracle's, everything else unchanged."""
    w = W.make_prefill("app", seed=8, batch=4, hq=8, hkv=8, d=128, dtype="bf16",
                       hist=[100, 0, 4000, 33], chunk=[512, 512, 512, 512])
    w.slots[7] = -1
    d = to_dev(w, DEV)
    pkv.kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"])
    torch.cuda.synchronize()
    pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
    assert torch.equal(bits(d["k_cache"]), bits(w.k_cache))
    assert torch.equal(bits(d["v_cache"]), bits(w.v_cache))


# ------------------------------------------------------------- invariances

def test_page_permutation_bit_identical():
    w = W.make_decode("perm", seed=11, batch=6, hq=16, hkv=2, d=128, dtype="f16",
                      hist_lens=[5000, 77, 4096, 1, 2048, 3000], append=True, pool_slack=0.2)
    w2 = W.permute_pages(w, seed=99)
    for split in (0, 256):
        a, la = gpu_decode(w, to_dev(w, DEV), split)
        b, lb = gpu_decode(w2, to_dev(w2, DEV), split)
        assert torch.equal(bits(a), bits(b)) and torch.equal(bits(la), bits(lb))


def test_shared_prefix_equals_duplicated_bit_identical():
    w = W.make_decode("pfx", seed=12, batch=12, hq=32, hkv=8, d=128, dtype="bf16",
                      hist_lens=[2048 + s for s in (32, 100, 511, 64, 250, 33, 400, 1, 2, 17,
                                                     480, 300)],
                      append=False, shared_prefix=2048)
    w2 = W.duplicate_shared_pages(w)
    a, la = gpu_decode(w, to_dev(w, DEV))
    b, lb = gpu_decode(w2, to_dev(w2, DEV))
    assert torch.equal(bits(a), bits(b)) and torch.equal(bits(la), bits(lb))


def test_run_to_run_deterministic():
    w = W.make("llama8b")
    d = to_dev(w, DEV)
    pkv.kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"])
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"],
            w.max_context_len, w.scale)
    a = pkv.paged_attn_decode(*args, split_tokens=512)
    b = pkv.paged_attn_decode(*args, split_tokens=512)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))


def test_split_sweep_and_partials_path():
    """Every split size stays within tolerance of the oracle, and the two-call
    path (partials, then merge_states) is bit-identical to the one-call path."""
    w = W.make_decode("sweep", seed=13, batch=4, hq=16, hkv=2, d=128, dtype="f16",
                      hist_lens=[20000, 9000, 1, 16383], append=True)
    d = to_dev(w, DEV)
    pkv.kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"])
    ref, ref_lse = oracle_decode(w)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"],
            w.max_context_len, w.scale)
    for split in (16, 48, 256, 1024, 4096, 0, 32768):
        out, lse = pkv.paged_attn_decode(*args, split_tokens=split, return_lse=True)
        o_parts, l_parts, _ = pkv.paged_attn_decode_partials(*args, split_tokens=split)
        out2, lse2 = pkv.merge_states(o_parts, l_parts, out_dtype=torch.float16, return_lse=True)
        torch.cuda.synchronize()
        assert_close(out.reshape(ref.shape), ref, "f16", f"split {split}")
        assert_lse_close(lse.reshape(-1), ref_lse, "f16", f"split {split}")
        n_split, _ = pkv.decode_plan(pkv.cache_desc(d["k_cache"]), 4, 16, w.max_context_len, split)
        if n_split > 1:
            assert torch.equal(bits(out2.view_as(out)), bits(out))
            assert torch.equal(bits(lse2.view_as(lse)), bits(lse))


@pytest.mark.parametrize("dtype,hq,hkv,window", [("f16", 16, 2, 0), ("bf16", 8, 2, 0),
                                                 ("bf16", 32, 4, 700), ("f32", 4, 2, 0)])
def test_uneven_batch_with_split_for_lens(dtype, hq, hkv, window):
    """Lengths from 1 key to 20K in one batch, decoded with the lengths-aware
    split (many splits for the long rows, one for the short)."""
    lens = [1, 5, 100, 3000, 20000, 777]
    d_ = 64 if dtype == "f32" else 128
    w = W.make_decode("uneven", seed=121 + hq, batch=len(lens), hq=hq, hkv=hkv, d=d_,
                      dtype=dtype, hist_lens=lens, append=False, pool_slack=0.1)
    d = to_dev(w, DEV)
    desc = pkv.cache_desc(d["k_cache"])
    opts = pkv.decode_opts(d["q"].dtype, d["k_cache"].dtype, window=window, sink=16)
    split = pkv.decode_split_for_lens(desc, hq, lens, opts)
    n_split, _ = pkv.decode_plan(desc, w.batch, hq, w.max_context_len, split, opts)
    assert n_split > 1
    out, lse = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                     d["context_lens"], w.max_context_len, w.scale,
                                     split_tokens=split, return_lse=True, window=window,
                                     sink=16 if window else 0)
    torch.cuda.synchronize()
    ref, ref_lse = pkvref.decode_ex(dtype, dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                                    w.context_lens, w.scale, window=window,
                                    sink=16 if window else 0, n_threads=host_threads())
    assert_close(out.reshape(ref.shape), ref, dtype, f"uneven {dtype} G{hq // hkv}")
    assert_lse_close(lse.reshape(-1), ref_lse, dtype, f"uneven {dtype} G{hq // hkv}")


def test_merge_states_matches_oracle():
    gen = torch.Generator().manual_seed(14)
    rows, n, dd = 37, 70, 128
    o = torch.randn(rows, n, dd, generator=gen)
    l = torch.randn(rows, n, generator=gen) * 5
    l[3, :] = float("-inf")                   # all parts empty
    l[5, ::3] = float("-inf")                 # some parts empty
    o[5, ::3] = float("nan")                  # ... whose o is never read
    out, lse = pkv.merge_states(o.to(DEV), l.to(DEV), out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    o64 = o.double().numpy()
    o64[5, ::3] = 0.0
    ref, ref_lse = pkvref.merge(o64, l.double().numpy())
    assert_close(out, ref, "f32", "merge")
    assert_lse_close(lse, ref_lse, "f32", "merge")
    assert torch.all(out[3] == 0) and torch.isneginf(lse[3])


# ------------------------------------------------ broken preconditions

@pytest.mark.parametrize("hq", [8, 16, 32])
def test_bad_page_id_and_length_poison_only_their_row(hq):
    w = W.make_decode("bad", seed=15, batch=4, hq=hq, hkv=2, d=128, dtype="bf16",
                      hist_lens=[300, 300, 300, 300], append=False, pool_slack=0.2)
    w.block_table[1, 3] = w.num_pages + 5          # out-of-range page id inside the length
    w.block_table[2, 0] = -1
    d = to_dev(w, DEV)
    d["context_lens"][3] = w.stride * 16 + 40     # longer than the table row
    for split in (0, 64):
        out, lse = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                         d["context_lens"], w.stride * 16, w.scale,
                                         split_tokens=split, return_lse=True)
        torch.cuda.synchronize()
        assert torch.isfinite(out[0].float()).all()
        for b in (1, 2, 3):
            assert torch.isnan(out[b].float()).all(), (split, b)


def test_prepared_calls_match_regular_calls():
    """The pre-marshalled calls the benchmark uses give bit-identical results."""
    w = W.make_decode("prep", seed=16, batch=4, hq=16, hkv=2, d=128, dtype="f16",
                      hist_lens=[3000, 17, 900, 4100], append=True)
    d = to_dev(w, DEV)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"],
            w.max_context_len, w.scale)
    k0, v0 = d["k_cache"].clone(), d["v_cache"].clone()
    pkv.kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"])
    ref_out, ref_lse = pkv.paged_attn_decode(*args, split_tokens=256, return_lse=True)
    torch.cuda.synchronize()
    d["k_cache"].copy_(k0)
    d["v_cache"].copy_(v0)
    o_parts, l_parts, ws = pkv.paged_attn_decode_partials(*args, split_tokens=256)
    out = torch.empty_like(d["q"])
    lse = torch.empty(4, 16, dtype=torch.float32, device=DEV)
    calls = [pkv.binding.prepare_kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"],
                                           d["slots"]),
             pkv.binding.prepare_decode_partials(*args, 256, ws),
             pkv.binding.prepare_merge_states(o_parts, l_parts, out, lse)]
    for _ in range(2):
        for c in calls:
            c()
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref_out)) and torch.equal(bits(lse), bits(ref_lse))


@pytest.mark.parametrize("split,window", [(0, 0), (256, 0), (0, 300)])
def test_prepared_decode_same_bits(split, window):
    """The decode call marshalled once (binding.prepare_decode) gives the bits
    of the plain call, one launch or partials + merge, with options or not;
    the tiny batch (at most 32 pages) is not split by the automatic plan."""
    w = W.make("tiny")
    d = to_dev(w, DEV)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"],
            w.max_context_len, w.scale)
    n_split, ws_bytes = pkv.decode_plan(pkv.cache_desc(d["k_cache"]), w.batch, w.num_q_heads,
                                        w.max_context_len, split)
    assert (n_split == 1) == (split == 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    want = pkv.paged_attn_decode(*args, split_tokens=split, window=window, sink=4 if window else 0)
    out = torch.empty_like(d["q"])
    pkv.binding.prepare_decode(*args, split, out, workspace=ws, window=window,
                               sink=4 if window else 0)()
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(want))
    ref, _ = pkvref.decode_ex(w.dtype, w.dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                              w.context_lens, w.scale, window=window, sink=4 if window else 0,
                              n_threads=host_threads())
    assert_close(out.reshape(ref.shape), ref, w.dtype, f"prepared split {split} window {window}")
