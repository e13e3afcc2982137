"""Shared test utilities: tolerances and device copies."""
import os

import numpy as np
import torch

# Tolerances: f32 inputs max-abs 1e-5; f16/bf16 inputs (fp32 accumulate)
# |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise; lse 1e-5 / 1e-3.
ATOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
RTOL = {"f32": 0.0, "f16": 1e-2, "bf16": 1e-2}
LSE_TOL = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def as_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def assert_close(got, ref, dtype: str, what: str = ""):
    g = as_f64(got).reshape(np.asarray(ref).shape)
    r = np.asarray(ref, dtype=np.float64)
    tol = ATOL[dtype] + RTOL[dtype] * np.abs(r)
    ok = np.abs(g - r) <= tol          # False where g is NaN
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} elements outside tolerance; "
                             f"first at {i}: got {g[i]!r} ref {r[i]!r}; "
                             f"max abs err {np.nanmax(np.abs(g - r))}")


def assert_lse_close(got, ref, dtype: str, what: str = ""):
    g = as_f64(got).reshape(np.asarray(ref).shape)
    r = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(g) & np.isneginf(r)
    with np.errstate(invalid="ignore"):          # -inf - -inf where both are empty rows
        ok = both_inf | (np.abs(g - r) <= LSE_TOL[dtype])
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what} lse: got {g[i]!r} ref {r[i]!r}")


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a tensor's bytes, for bit-exact comparisons."""
    t = t.detach().contiguous().cpu()
    return t.view({4: torch.int32, 2: torch.int16, 1: torch.uint8}[t.element_size()])


def to_dev(w, dev):
    """Device copies of a workload's tensors (dict)."""
    d = dict(k_cache=w.k_cache.to(dev), v_cache=w.v_cache.to(dev), q=w.q.to(dev),
             block_table=w.block_table.to(dev), context_lens=w.context_lens.to(dev))
    for name in ("k_new", "v_new", "slots", "q_indptr"):
        x = getattr(w, name)
        d[name] = None if x is None else x.to(dev)
    return d
