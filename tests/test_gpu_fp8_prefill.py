"""GPU parity of chunked prefill and mixed batches over fp8 pools (page 4,
section 3.1 prefills in chunks over an fp8_e5m2 cache; page 1, section 4.1
names e4m3) against the oracle, through the C ABI: the chunk's K/V go in by
the quantizing append (bytes compared with the oracle's quantizer), then the
MFMA prefill widens each page exactly to the query type.  Every output row
and log-sum-exp is compared within the 16-bit tolerances."""
import pytest
import torch

import paged_kv_cache_04_amd as pkv
from oracle import pkvref
from paged_kv_cache_04_amd import workloads as W

from helpers import assert_close, assert_lse_close, bits, host_threads, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SCALES = dict(k_scale=0.0234375, v_scale=0.01953125)


def gpu_append(w, d):
    pkv.kv_append_quant(d["k_cache"], d["v_cache"], d["k_new"], d["v_new"], d["slots"],
                        w.k_scale, w.v_scale)


def oracle_append(w):
    f8 = W.DTYPES[w.kv_dtype]
    kq = torch.from_numpy(pkvref.quant_fp8(w.kv_dtype, w.dtype, w.k_new, w.k_scale)).view(f8)
    vq = torch.from_numpy(pkvref.quant_fp8(w.kv_dtype, w.dtype, w.v_new, w.v_scale)).view(f8)
    pkvref.kv_append(w.kv_dtype, w.k_cache, w.v_cache, kq, vq, w.slots)


def oracle(w, rows=None):
    return pkvref.prefill_ex(w.dtype, w.kv_dtype, w.k_cache, w.v_cache, w.q, w.q_indptr,
                             w.block_table, w.context_lens, w.scale, k_scale=w.k_scale,
                             v_scale=w.v_scale, rows=rows, n_threads=host_threads())


def gpu_prefill(w, d):
    out, lse = pkv.paged_attn_prefill_chunk(d["q"], d["k_cache"], d["v_cache"], d["q_indptr"],
                                            d["block_table"], d["context_lens"],
                                            max(w.meta["chunk_lens"]), w.max_context_len,
                                            w.scale, return_lse=True, k_scale=w.k_scale,
                                            v_scale=w.v_scale)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    ("fp8_e4m3", "f16", 16, 2, [0, 100, 1000], [300, 64, 129]),    # G 8
    ("fp8_e5m2", "bf16", 32, 8, [0, 777, 2000], [77, 256, 129]),   # G 4
    ("fp8_e5m2", "f16", 32, 2, [5, 500], [600, 33]),               # G 16
    ("fp8_e4m3", "bf16", 8, 4, [63, 64, 65], [1, 2, 200]),         # G 2, tile edges
    ("fp8_e4m3", "f16", 8, 8, [0, 16], [16, 47]),                  # G 1
]


@pytest.mark.parametrize("kv,qd,hq,hkv,hist,chunk", CASES)
def test_fp8_prefill_all_rows(kv, qd, hq, hkv, hist, chunk):
    w = W.make_prefill("f8p", seed=hq + 7 * hkv + len(hist), batch=len(hist), hq=hq, hkv=hkv,
                       d=128, dtype=qd, hist=hist, chunk=chunk, pool_slack=0.2, kv_dtype=kv,
                       **SCALES)
    d = to_dev(w, DEV)
    gpu_append(w, d)
    out, lse = gpu_prefill(w, d)
    oracle_append(w)
    assert torch.equal(bits(d["k_cache"]), bits(w.k_cache)), "k pool after quantizing append"
    assert torch.equal(bits(d["v_cache"]), bits(w.v_cache)), "v pool after quantizing append"
    ref, ref_lse = oracle(w)
    what = f"fp8 prefill {kv}/{qd} G{hq // hkv}"
    assert_close(out.reshape(ref.shape), ref, qd, what)
    assert_lse_close(lse.reshape(-1), ref_lse, qd, what)


def test_fp8_prefill_one_row_chunks_match_fp8_decode():
    """A chunk of one row at the end of its sequence is a decode row: the
    prefill kernel and the fp8 decode kernel agree within tolerance, and both
    match the oracle."""
    w = W.make_prefill("f8r", seed=5, batch=4, hq=16, hkv=2, d=128, dtype="f16",
                       hist=[0, 15, 700, 3000], chunk=[1, 1, 1, 1], pool_slack=0.2,
                       kv_dtype="fp8_e5m2", **SCALES)
    d = to_dev(w, DEV)
    gpu_append(w, d)
    out, lse = gpu_prefill(w, d)
    dq = d["q"].view(w.batch, w.num_q_heads, w.head_dim)
    dout, dlse = pkv.paged_attn_decode(dq, d["k_cache"], d["v_cache"], d["block_table"],
                                       d["context_lens"], w.max_context_len, w.scale,
                                       return_lse=True, **SCALES)
    torch.cuda.synchronize()
    oracle_append(w)
    ref, ref_lse = oracle(w)
    assert_close(out.reshape(ref.shape), ref, "f16", "prefill rows")
    assert_close(dout.reshape(ref.shape), ref, "f16", "decode rows")
    assert_lse_close(lse.reshape(-1), ref_lse, "f16", "prefill rows")
    assert_close(out.reshape(ref.shape).float(), dout.reshape(ref.shape).float().cpu().numpy(),
                 "f16", "prefill vs decode")


@pytest.mark.parametrize("kv,qd,hq,hkv", [("fp8_e4m3", "f16", 16, 2), ("fp8_e5m2", "bf16", 32, 8),
                                          ("fp8_e5m2", "f16", 32, 2)])
def test_fp8_mixed_batch_all_rows(kv, qd, hq, hkv):
    w = W.make_mixed("f8m", seed=hq + hkv, hq=hq, hkv=hkv, d=128, dtype=qd,
                     decode_hist=[0, 15, 16, 300, 1000], chunk_hist=[0, 37, 500],
                     chunk=[7, 129, 64], pool_slack=0.2, kv_dtype=kv, **SCALES)
    d = to_dev(w, DEV)
    gpu_append(w, d)
    nd = w.meta["num_decode"]
    out, lse = pkv.paged_attn_mixed(d["q"], d["k_cache"], d["v_cache"], d["q_indptr"],
                                    d["block_table"], d["context_lens"], nd,
                                    max(w.meta["chunk_lens"]), w.max_context_len, w.scale,
                                    split_tokens=256, return_lse=True, **SCALES)
    torch.cuda.synchronize()
    oracle_append(w)
    ref, ref_lse = oracle(w)
    what = f"fp8 mixed {kv}/{qd} G{hq // hkv}"
    assert_close(out.reshape(ref.shape), ref, qd, what)
    assert_lse_close(lse.reshape(-1), ref_lse, qd, what)


def test_fp8_prefill_full_size_sampled():
    """The prefill shape (batch 4, 32768 + 512, 32 / 8 heads) over e5m2
    pools: sampled rows of every sequence against the oracle."""
    w = W.make("prefill_fp8")
    print("[fp8 prefill parity] 4 x (32768 + 512), e5m2", flush=True)
    d = to_dev(w, DEV)
    gpu_append(w, d)
    out, lse = gpu_prefill(w, d)
    oracle_append(w)
    hq = w.num_q_heads
    ind = w.q_indptr.tolist()
    rows = []
    for b in range(w.batch):
        for i in (0, 1, 63, 64, 255, 256, 511):
            for h in (0, 5, 31):
                rows.append((ind[b] + i) * hq + h)
    ref, ref_lse = oracle(w, rows=rows)
    got = out.reshape(-1, w.head_dim)[rows]
    assert_close(got, ref, w.dtype, "fp8 prefill 32K")
    assert_lse_close(lse.reshape(-1)[rows], ref_lse, w.dtype, "fp8 prefill 32K")


def test_fp8_prefill_zero_keys_and_constant_values():
    """Closed forms over fp8 pools: all-zero keys give the running mean of
    the visible V rows (times v_scale); constant V rows give that constant."""
    import numpy as np
    hist, chunk = [0, 90, 700], [70, 33, 129]
    for what in ("zero K", "constant V"):
        w = W.make_prefill("f8z", seed=19, batch=3, hq=16, hkv=2, d=128, dtype="bf16",
                           hist=hist, chunk=chunk, pool_slack=0.2, kv_dtype="fp8_e4m3",
                           k_scale=0.03125, v_scale=0.0625)
        f8 = W.DTYPES["fp8_e4m3"]
        if what == "zero K":
            k = torch.zeros(w.k_cache.shape, dtype=torch.float32).to(f8)
            k.view(torch.uint8)[w.k_cache.view(torch.uint8) == 0x7F] = 0x7F
            w.k_cache, w.k_new = k, torch.zeros_like(w.k_new)
        else:
            v = torch.full(w.v_cache.shape, -1.5 / w.v_scale).to(f8)   # -24: exact in e4m3
            v.view(torch.uint8)[w.v_cache.view(torch.uint8) == 0x7F] = 0x7F
            w.v_cache, w.v_new = v, torch.full_like(w.v_new, -1.5)
        d = to_dev(w, DEV)
        gpu_append(w, d)
        out, _ = gpu_prefill(w, d)
        if what == "constant V":
            assert_close(out, np.full(tuple(out.shape), -1.5), "bf16", "fp8 prefill constant V")
            continue
        oracle_append(w)
        G = w.num_q_heads // w.num_kv_heads
        row = 0
        for b in range(3):
            n = hist[b] + chunk[b]
            pages = w.meta["page_lists"][b]
            vr = torch.stack([w.v_cache[pages[t // 16], :, t % 16, :].to(torch.float64)
                              for t in range(n)]) * w.v_scale          # [n][H_kv][D]
            mean = torch.cumsum(vr, 0) / torch.arange(1, n + 1, dtype=torch.float64)[:, None, None]
            for i in range(chunk[b]):
                want = mean[hist[b] + i].repeat_interleave(G, dim=0).numpy()
                assert_close(out[row], want, "bf16", f"fp8 prefill zero K b{b} row {i}")
                row += 1


def test_fp8_prefill_bad_page_poisons_its_rows_only():
    """A block-table entry outside the pool makes every row of its sequence
    NaN (and its log-sum-exp NaN); the other sequence is untouched."""
    w = W.make_prefill("f8bad", seed=29, batch=2, hq=16, hkv=2, d=128, dtype="bf16",
                       hist=[200, 200], chunk=[40, 40], pool_slack=0.2, kv_dtype="fp8_e5m2",
                       **SCALES)
    d = to_dev(w, DEV)
    gpu_append(w, d)
    d["block_table"][1, 2] = w.num_pages + 3
    out, lse = gpu_prefill(w, d)
    assert torch.isfinite(out[:40].float()).all() and torch.isfinite(lse[:40]).all()
    assert torch.isnan(out[40:].float()).all() and torch.isnan(lse[40:]).all()
