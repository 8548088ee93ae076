"""Helpers shared by the GPU parity tests: run a synthetic step through the C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np

from oracle import reference as R
from synth import LayerSpec, Request, Workload

# tolerances against the fp64 oracle: fp32 path max-abs; bf16 paths max-abs and mean-abs (fp32 accumulation)
TOL_F32_MAX = 1e-5
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3


def gpu_rows(step, layer, tokens):
    import torch
    out = step.layers[layer].out
    idx = torch.as_tensor(np.asarray(tokens, dtype=np.int64), device=out.device)
    return out.index_select(0, idx).float().cpu().numpy().astype(np.float64)


def compare(w, step, layer, tokens=None, label=""):
    """Max/mean abs error of the GPU rows against the oracle (all rows, or `tokens`). Asserts the tolerance."""
    sched = R.schedule(w)
    # the device ran the library's schedule; it must be the oracle's (checked bit-exactly elsewhere)
    assert np.array_equal(sched["query_start_loc"], step.sched["query_start_loc"])
    assert np.array_equal(sched["seq_lens"], step.sched["seq_lens"])
    if tokens is None:
        tokens = list(range(sched["num_tokens"]))
    tokens = sorted(set(int(t) for t in tokens))
    ref = R.rows_reference(w, layer, sched, tokens)
    want = np.stack([ref[t] for t in tokens])
    got = gpu_rows(step, layer, tokens)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    if w.dtype == "f32":
        assert mx <= TOL_F32_MAX, f"{label}: max abs {mx:.3g} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, f"{label}: max {mx:.3g} mean {mean:.3g}"
    return mx, mean


def logical_cache(step, layer):
    """Device caches read back as logical [page, offset, Hkv, D] float32."""
    L = step.layers[layer]
    k = L.k_cache.float().cpu().numpy().transpose(0, 2, 1, 3)
    v = L.v_cache.float().cpu().numpy().transpose(0, 3, 1, 2)
    return k, v


def same_bits(a, b):
    """Equal as float32 values, NaN positions included."""
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na], b[~nb])


def custom_workload(requests, *, Hq=8, Hkv=2, D=128, P=16, dtype="bf16", budget=4096, window_left=-1,
                    ring_len=0, n_pages=None, seed=77, name="custom"):
    """A one-layer workload from explicit requests (state, computed, pending); pages are drawn from a shuffled pool."""
    rng = np.random.default_rng(seed)
    reqs = []
    need = 0
    for i, (st, comp, pend) in enumerate(requests):
        reqs.append(Request(i, st, comp, pend, [None]))
        need += ring_len if ring_len else -(-(comp + pend) // P)
    n_alloc = n_pages or max(8, int(need * 1.3) + 4)
    order = (rng.permutation(n_alloc) + 2).astype(np.int32)
    pos = 0
    for rq in reqs:
        c = (ring_len if rq.state != 2 else 0) if ring_len else -(-rq.num_computed // P)
        rq.pages[0] = order[pos:pos + c].copy()
        pos += c
    lay = LayerSpec("sliding" if ring_len else "full", 0, window_left, ring_len, n_alloc + 2, (0, 1), order[pos:])
    return Workload(name, 0, seed, dtype, Hq, Hkv, D, P, 1.0 / np.sqrt(D), budget, 4096, 0.0, [lay], reqs)
