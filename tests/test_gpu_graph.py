"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph): the
host layer only launches kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a captured decode step, prefill call or
mixed-batch call replays to the eager result bit for bit.  Each graph is
replayed several times with eager library work and synchronisations in
between, and every replay is compared."""
import pytest
import torch

import paged_kv_cache_04_amd as pkv
from paged_kv_cache_04_amd import binding as B
from paged_kv_cache_04_amd import workloads as W

from helpers import bits, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def replay_matches(graph, outputs, eager, other_work, reps=4):
    for r in range(reps):
        for o in outputs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, eager):
            assert torch.equal(bits(got), bits(want)), f"replay {r}"
        other_work()
        torch.cuda.synchronize()


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hq", [8, 16])
def test_decode_step_graph(hq, fused):
    """append + split-KV partials + merge, as the decode step runs: three
    launches, or two when the partial launch stores the new tokens."""
    w = W.make_decode("gr", seed=101 + hq, batch=4, hq=hq, hkv=2, d=128, dtype="f16",
                      hist_lens=[100, 1000, 3000, 5000], append=True, pool_slack=0.1)
    d = to_dev(w, DEV)
    dargs = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["context_lens"],
             w.max_context_len, w.scale)
    n_split, _ = pkv.decode_plan(pkv.cache_desc(d["k_cache"]), w.batch, w.num_q_heads,
                                 w.max_context_len, 256)
    assert n_split > 1
    _, total = B.partials_bytes(w.batch, w.num_q_heads, n_split, w.head_dim)
    ws = torch.empty(total, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    o_parts, l_parts, _ = pkv.paged_attn_decode_partials(*dargs, split_tokens=256, workspace=ws)

    def step_calls():
        merge = B.prepare_merge_states(o_parts, l_parts, out, lse)
        if fused:
            return (B.prepare_decode_append_partials(d["q"], d["k_cache"], d["v_cache"],
                                                     d["k_new"], d["v_new"], d["block_table"],
                                                     d["context_lens"], w.max_context_len,
                                                     w.scale, 256, ws), merge)
        return (B.prepare_kv_append(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"],
                                    d["slots"]),
                B.prepare_decode_partials(*dargs, 256, ws), merge)

    for c in step_calls():
        c()
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone(), d["k_cache"].clone(), d["v_cache"].clone())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in step_calls():       # prepared on the capture stream
            c()
    other = torch.empty_like(out)

    def other_work():
        pkv.paged_attn_decode(*dargs, split_tokens=0, out=other)

    replay_matches(g, (out, lse), eager[:2], other_work)
    # the replays stored the same rows again: the pools are as after the eager step
    assert torch.equal(bits(d["k_cache"]), bits(eager[2]))
    assert torch.equal(bits(d["v_cache"]), bits(eager[3]))


def test_prefill_and_mixed_graph():
    wp = W.make_prefill("grp", seed=111, batch=3, hq=16, hkv=2, d=128, dtype="bf16",
                        hist=[0, 500, 2000], chunk=[300, 64, 129], pool_slack=0.1)
    dp = to_dev(wp, DEV)
    pkv.kv_append(dp["k_cache"], dp["v_cache"], dp["k_new"], dp["v_new"], dp["slots"])
    out = torch.empty_like(dp["q"])
    lse = torch.empty((dp["q"].shape[0], wp.num_q_heads), dtype=torch.float32, device=DEV)
    args = (dp["q"], dp["k_cache"], dp["v_cache"], dp["q_indptr"], dp["block_table"],
            dp["context_lens"], max(wp.meta["chunk_lens"]), wp.max_context_len, wp.scale)
    pkv.paged_attn_prefill_chunk(*args, out=out, lse_out=lse)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.paged_attn_prefill_chunk(*args, out=out, lse_out=lse)
    replay_matches(g, (out, lse), eager,
                   lambda: pkv.paged_attn_prefill_chunk(*args, out=torch.empty_like(out)))

    wm = W.make_mixed("grm", seed=112, hq=16, hkv=2, d=128, dtype="f16",
                      decode_hist=[5, 900, 4000], chunk_hist=[0, 300], chunk=[70, 200],
                      pool_slack=0.1)
    dm = to_dev(wm, DEV)
    pkv.kv_append(dm["k_cache"], dm["v_cache"], dm["k_new"], dm["v_new"], dm["slots"])
    nd = wm.meta["num_decode"]
    n_split, ws_bytes = pkv.decode_plan(pkv.cache_desc(dm["k_cache"]), nd, wm.num_q_heads,
                                        wm.max_context_len, 512)
    assert n_split > 1
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    mout = torch.empty_like(dm["q"])
    margs = (dm["q"], dm["k_cache"], dm["v_cache"], dm["q_indptr"], dm["block_table"],
             dm["context_lens"], nd, 200, wm.max_context_len, wm.scale)
    pkv.paged_attn_mixed(*margs, split_tokens=512, out=mout, workspace=ws)
    torch.cuda.synchronize()
    eager_m = (mout.clone(),)
    gm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gm):
        pkv.paged_attn_mixed(*margs, split_tokens=512, out=mout, workspace=ws)
    replay_matches(gm, (mout,), eager_m,
                   lambda: pkv.paged_attn_mixed(*margs, split_tokens=0,
                                                out=torch.empty_like(mout)))


def test_shared_prefix_graph():
    """The shared-prefix decode (three launches: the shared pages on the
    matrix cores, the own pages on the split-KV decode, the merge), captured
    on torch's capture stream: every replay gives the eager result bit for
    bit."""
    prefix, suffix = 512, [3, 200, 1000, 64]
    w = W.make_decode("grs", seed=113, batch=len(suffix), hq=32, hkv=8, d=128, dtype="bf16",
                      hist_lens=[prefix + s for s in suffix], append=False, pool_slack=0.1,
                      shared_prefix=prefix)
    d = to_dev(w, DEV)
    pp = prefix // 16
    prefix_table = d["block_table"][0, :pp].contiguous()
    own = d["block_table"][:, pp:].contiguous()
    suffix_lens = (d["context_lens"] - prefix).contiguous()
    max_suffix = int(suffix_lens.max().item())
    n_parts, ws_bytes = pkv.shared_prefix_plan(pkv.cache_desc(d["k_cache"]), w.batch,
                                               w.num_q_heads, prefix, max_suffix)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=DEV)
    args = (d["q"], d["k_cache"], d["v_cache"], prefix_table, prefix, own, suffix_lens,
            max_suffix, w.scale)
    pkv.paged_attn_decode_shared_prefix(*args, out=out, lse_out=lse, workspace=ws)
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.paged_attn_decode_shared_prefix(*args, out=out, lse_out=lse, workspace=ws)
    ws2 = torch.empty_like(ws)
    replay_matches(g, (out, lse), eager,
                   lambda: pkv.paged_attn_decode_shared_prefix(*args, out=torch.empty_like(out),
                                                               workspace=ws2))
