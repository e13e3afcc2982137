"""Seeded workload generators: determinism and pool invariants."""
import torch

from paged_kv_cache_04_amd import workloads as W


def test_same_seed_same_bytes():
    a = W.make_decode("a", seed=7, batch=3, hq=4, hkv=2, d=16, dtype="bf16",
                      hist_lens=[5, 40, 17], append=True, pool_slack=0.1)
    b = W.make_decode("a", seed=7, batch=3, hq=4, hkv=2, d=16, dtype="bf16",
                      hist_lens=[5, 40, 17], append=True, pool_slack=0.1)
    for x, y in ((a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.q, b.q),
                 (a.k_new, b.k_new)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(a.block_table, b.block_table) and torch.equal(a.slots, b.slots)


def test_pool_invariants_tiny():
    w = W.make("tiny")
    assert w.num_pages == 128 and w.head_dim == 64 and w.dtype == "f32"
    assert w.context_lens.tolist() == [37, 128, 200, 511]
    used = set()
    for b, pl in enumerate(w.meta["page_lists"]):
        L = int(w.context_lens[b])
        assert len(pl) == W.pages_for(L)                     # ceil(L / P) pages
        assert list(w.block_table[b, : len(pl)]) == pl
        assert all(int(x) == w.poison_page for x in w.block_table[b, len(pl):])
        used.update(pl)
        # stored rows finite, tail of the last page NaN (valid_length <= P)
        last = pl[-1]
        fill = L - (len(pl) - 1) * W.PAGE_SIZE
        assert 0 < fill <= W.PAGE_SIZE
        assert torch.isfinite(w.k_cache[last, :, :fill]).all()
        assert torch.isnan(w.k_cache[last, :, fill:]).all()
    assert len(used) == 56
    assert w.poison_page not in used and torch.isnan(w.k_cache[w.poison_page]).all()
    # pages are not in order (non-contiguous placement)
    assert w.meta["page_lists"][3] != sorted(w.meta["page_lists"][3])


def test_append_slot_is_next_position():
    w = W.make_decode("s", seed=3, batch=4, hq=4, hkv=2, d=16, dtype="f16",
                      hist_lens=[15, 16, 31, 1], append=True)
    for b in range(4):
        h = w.meta["hist_lens"][b]
        pl = w.meta["page_lists"][b]
        s = int(w.slots[b])
        assert s // W.PAGE_SIZE == pl[h // W.PAGE_SIZE] and s % W.PAGE_SIZE == h % W.PAGE_SIZE
        assert torch.isnan(w.k_cache[s // 16, :, s % 16]).all()   # empty until appended
        assert int(w.context_lens[b]) == h + 1


def test_shared_prefix_pages_in_every_table():
    w = W.make_decode("p", seed=4, batch=6, hq=4, hkv=2, d=16, dtype="bf16",
                      hist_lens=[32 + 5] * 6, append=False, shared_prefix=32)
    pre = w.block_table[:, :2]
    assert (pre == pre[0]).all()
    d = W.duplicate_shared_pages(w)
    assert len(set(d.block_table[:, 0].tolist())) == 6


def test_prefill_workload_layout():
    w = W.make_prefill("f", seed=5, batch=2, hq=4, hkv=2, d=16, dtype="bf16",
                       hist=[20, 0], chunk=[7, 3])
    assert w.q.shape == (10, 4, 16)
    assert w.q_indptr.tolist() == [0, 7, 10]
    assert w.context_lens.tolist() == [27, 3]
    assert w.slots.shape == (10,)
