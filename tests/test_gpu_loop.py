"""GPU parity of a serving loop: steps whose schedules differ from one step to the next.

The package's pipeline schedules every step from the current request state (cb_build_metadata), the harness writes
the step's new Q/K/V rows, the kernels run, and the request lifecycle moves on (cb_advance, in place on the
scheduler's state): decodes grow their
context by one key per step, prefill chunks continue, a waiting prompt is admitted and prefilled in chunks, then
decodes. Every step is checked against the oracle run on the same request state, in three modes: the metadata copy
on its own stream (eager launches), graph replay by padded shape, and per-phase launches between timing events.
Consecutive steps use the two metadata buffer pairs alternately and differ, so a step that read the other pair or
stale metadata fails. Tolerances as in the other parity tests (bf16 max-abs 2e-2, mean-abs 2e-3; pages bit-exact).
"""
import dataclasses

import numpy as np
import pytest

from oracle import reference as R
from synth import make_workload
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MODES = ["copy stream", "graph replay", "per-phase launches with events"]


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_varlen_amd import load_library
    load_library()
    return torch


def _state(w, sched_obj):
    """The workload as the oracle sees it at the scheduler's current request state."""
    layers = [dataclasses.replace(lay, free_pages=f) for lay, f in zip(w.layers, sched_obj.free_pages)]
    return dataclasses.replace(w, requests=list(sched_obj.requests), layers=layers)


def _loop(torch, w, steps, mode, rows, sample=None, seed=0):
    from harness import build_step, pipeline_for, upload_new_rows
    from paged_kv_attention_varlen_amd.hip_events import HipEvent
    st = build_step(w, rows=rows, workspace_bytes=64 << 20)
    pipe = pipeline_for(w, st, graphs=(mode == "graph replay"))
    pipe.keep_schedule = True
    events = None
    if mode.startswith("per-phase"):
        events = [[HipEvent(timing=True, system_fence=False) for _ in range(6)] for _ in w.layers]
    rng = np.random.default_rng(seed)
    shapes = set()
    for k in range(steps):
        wk = _state(w, pipe.sched)                     # the request state this step is scheduled from
        views = pipe.prepare()
        s = pipe.last_schedule
        upload_new_rows(wk, s, st)
        for L in st.layers:
            L.out.fill_(float("nan"))
        pipe.launch(views, events)
        torch.cuda.synchronize()
        shapes.add(pipe.key)
        ref_sched = R.schedule(wk)
        assert np.array_equal(ref_sched["query_start_loc"], s["query_start_loc"]), f"step {k}: schedule differs"
        assert np.array_equal(ref_sched["seq_lens"], s["seq_lens"]), f"step {k}: schedule differs"
        T = s["num_tokens"]
        toks = list(range(T))
        if sample is not None and T > sample:
            qsl, seq = s["query_start_loc"], s["seq_lens"]
            nd = s["num_decodes"]
            pick = {int(qsl[int(np.argmax(seq[:nd]))])} if nd else set()
            pick |= {int(x) for x in rng.choice(T, size=sample, replace=False)}
            toks = sorted(pick)
        for l, L in enumerate(st.layers):
            out = L.out[:T].float()
            assert bool(torch.isfinite(out).all()), f"step {k} layer {l}: non-finite output"
            ref = R.rows_reference(wk, l, ref_sched, toks)
            want = np.stack([ref[t] for t in toks])
            got = out[torch.as_tensor(toks, device=out.device)].cpu().numpy().astype(np.float64)
            err = np.abs(got - want)
            assert err.max() <= H.TOL_BF16_MAX and err.mean() <= H.TOL_BF16_MEAN, \
                f"{mode} {w.name} step {k} layer {l}: max {err.max():.3g} mean {err.mean():.3g}"
            touched = sorted(set((s["layers"][l]["slot_mapping"] // w.page_size).tolist()))[:48]
            ids, k_ref, v_ref = R.pages_reference(wk, l, ref_sched, touched)
            kc, vc = H.logical_cache(st, l)
            assert H.same_bits(kc[ids], k_ref) and H.same_bits(vc[ids], v_ref), f"step {k} layer {l}: pages"
        if events is not None:
            for l in range(len(w.layers)):
                assert events[l][0].elapsed_time(events[l][1]) >= 0.0
        print(f"[gpu] {mode} step {k}: T={T} N={s['num_reqs']} decodes={s['num_decodes']} key={pipe.key}",
              flush=True)
        pipe.advance()
    return pipe, shapes


@pytest.mark.parametrize("mode", MODES)
def test_decode_loop_growing_contexts(torch_gpu, mode):
    """The full-size decode-only step run as 16 decode steps: every context grows by one key per step, requests
    cross page boundaries and take fresh pages. With graph replay the step pads to one or two shapes, so a handful
    of graphs serve all 16 steps."""
    w = make_workload(2)
    pipe, shapes = _loop(torch_gpu, w, 16, mode, rows=64, sample=12, seed=2)
    if mode == "graph replay":
        print(f"[gpu] decode loop: {len(shapes)} padded shapes, {pipe.captures} captures, {pipe.replays} replays",
              flush=True)
        assert pipe.replays == 16
        assert pipe.captures == len(shapes) <= 4


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("idx", [3, 5])
def test_chunk_progression(torch_gpu, idx, mode):
    """The reduced mixed step and hybrid layer pair run for 10 steps: continuing chunks finish and start decoding,
    the waiting prompt is admitted and prefilled in chunks, the token count and the plans change every step. All
    rows of every step are checked."""
    w = make_workload(idx, mini=True)
    pipe, shapes = _loop(torch_gpu, w, 10, mode, rows=w.max_batch_tokens, seed=idx)
    if mode == "graph replay":
        assert pipe.replays == 10
        assert pipe.captures == len(shapes) and len(pipe.graphs) <= pipe.max_graphs


def test_graph_cache_stays_bounded(torch_gpu):
    """More padded shapes than the cache holds: the least recently used graphs are evicted, the count stays at the
    bound, and replays stay correct (checked above on every step)."""
    w = make_workload(3, mini=True)
    from harness import build_step, pipeline_for, upload_new_rows
    st = build_step(w, rows=w.max_batch_tokens, workspace_bytes=64 << 20)
    pipe = pipeline_for(w, st, graphs=True, max_graphs=2, q_interval=16, item_interval=8)
    pipe.keep_schedule = True
    for k in range(8):
        wk = _state(w, pipe.sched)
        views = pipe.prepare()
        upload_new_rows(wk, pipe.last_schedule, st)
        pipe.launch(views)
        torch_gpu.cuda.synchronize()
        assert len(pipe.graphs) <= 2
        pipe.advance()
    assert pipe.captures > 2


def test_hybrid_pair_full_size_loop(torch_gpu):
    """The hybrid layer pair at full size (8192-token budget, full and sliding layers) as a three-step serving loop
    replaying graphs by padded shape (eager loops run at full size for the decode-only step and at reduced size for
    the layer pair above): the native lifecycle moves the 128 decodes, the continuing chunks and the new prompt on
    between steps, and each step's plans (the largest of the workloads) replace the last. Per step and layer: the
    longest decode row and 24 random rows against the oracle on the same request state, 48 of the pages the append
    touched bit for bit, and every output row finite."""
    w = make_workload(5)
    pipe, shapes = _loop(torch_gpu, w, 3, "graph replay", rows=w.max_batch_tokens, sample=24, seed=55)
    assert pipe.replays == 3 and pipe.captures == len(shapes)
