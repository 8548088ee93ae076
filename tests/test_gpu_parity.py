"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Reduced workloads are compared element by element on every output row and every cache page. At full size, in the
launch configuration the benchmark times: every row and every touched page of the decode-only step, the mixed
2048-token step and the large decode batch; for the hybrid layer pair, every row of every split prefill tile, three
unsplit tiles, a strided sample and decode rows, plus every touched page. Tolerances: fp32 max-abs 1e-5; bf16
max-abs 2e-2 and mean-abs 2e-3; append bit-exact.
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import reference as R
from synth import DECODING, PREFILLING, WAITING, make_workload
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_varlen_amd import load_library
    load_library()
    return torch


def _run(w, fused=False, **kw):
    """Build the step and run it: cb_kv_append then cb_paged_attention, or (fused) cb_paged_attention alone with the
    new K/V passed in, appending them itself."""
    from harness import build_step
    print(f"[gpu] {w.name} fused={fused} {kw}", flush=True)
    st = build_step(w, **kw)
    st.run(fused_append=fused)
    import torch
    torch.cuda.synchronize()
    return st


def _check_pages(w, st, layer, pages=None):
    ids, k_ref, v_ref = R.pages_reference(w, layer, R.schedule(w), pages)
    k, v = H.logical_cache(st, layer)
    assert H.same_bits(k[ids], k_ref), "K cache differs"
    assert H.same_bits(v[ids], v_ref), "V cache differs"


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_reduced_workload_all_rows_and_pages(torch_gpu, idx, fused):
    w = make_workload(idx, mini=True)
    st = _run(w, fused=fused)
    for l in range(len(w.layers)):
        mx, mean = H.compare(w, st, l, label=f"w{idx} reduced layer {l}")
        print(f"  layer {l}: max {mx:.3g} mean {mean:.3g}", flush=True)
        _check_pages(w, st, l)


@pytest.mark.parametrize("idx", [3, 5])
def test_reduced_workload_wide_prefill_tiles(torch_gpu, idx):
    """The reduced mixed step and layer pair with 256-row prefill tiles (8-wave work groups) forced: every row and
    every page."""
    w = make_workload(idx, mini=True)
    st = _run(w, fused=True, prefill_rows=256)
    G = w.Hq // w.Hkv
    assert all(L.plan.info.prefill_tokens * G == 256 for L in st.layers if L.plan.info.n_prefill)
    for l in range(len(w.layers)):
        mx, mean = H.compare(w, st, l, label=f"w{idx} reduced layer {l}")
        print(f"  layer {l}: max {mx:.3g} mean {mean:.3g}", flush=True)
        _check_pages(w, st, l)


def _sample_tokens(sched, rng, n_dec=12, per_chunk=6):
    qsl = sched["query_start_loc"]
    seq = sched["seq_lens"]
    nd = sched["num_decodes"]
    toks = set()
    if nd:
        dec = np.arange(nd)
        toks |= {int(qsl[int(np.argmax(seq[:nd]))]), int(qsl[int(np.argmin(seq[:nd]))])}
        toks |= {int(qsl[r]) for r in rng.choice(dec, size=min(n_dec, nd), replace=False)}
    for r in range(nd, sched["num_reqs"]):
        a, b = int(qsl[r]), int(qsl[r + 1])
        toks |= {a, b - 1}
        toks |= {int(t) for t in rng.integers(a, b, size=min(per_chunk, b - a))}
    return sorted(toks)


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_full_workload_every_row_and_touched_page(torch_gpu, idx):
    """The decode-only step, the mixed 2048-token step and the large decode batch at full size, in the launch
    configuration the benchmark times (the append fused into the decode launch): every output row element by
    element, and every page the step's append wrote, bit for bit."""
    w = make_workload(idx)
    st = _run(w, fused=True)
    sched = R.schedule(w)
    out = st.layers[0].out
    assert bool(torch_gpu.isfinite(out.float()).all()), "non-finite output somewhere"
    mx, mean = H.compare(w, st, 0, label=f"w{idx} full")
    print(f"  all {sched['num_tokens']} rows: max {mx:.3g} mean {mean:.3g}", flush=True)
    touched = sorted(set((sched["layers"][0]["slot_mapping"] // w.page_size).tolist()))
    _check_pages(w, st, 0, touched)
    print(f"  {len(touched)} touched pages bit-exact", flush=True)


def _tile_rows(plan, qsl_tokens, want_split, limit=None):
    """Token rows of prefill tiles: those cut into several key-range items (want_split) or not."""
    items = plan.items("prefill")
    count = {}
    for it in items:
        count[(int(it[1]), int(it[3]))] = count.get((int(it[1]), int(it[3])), 0) + 1
    tiles = sorted(k for k, n in count.items() if (n > 1) == want_split)
    if limit is not None and len(tiles) > limit:
        pick = np.linspace(0, len(tiles) - 1, limit).round().astype(int)
        tiles = [tiles[i] for i in pick]
    return sorted({t0 + i for t0, qc in tiles for i in range(qc)}), len(tiles)


def test_full_hybrid_pair_split_tiles_and_strided_rows(torch_gpu):
    """The hybrid layer pair at full size (8192 tokens, both layers), as the benchmark runs it. Per layer: every row
    of every prefill tile whose key range the plan cut into several items (their partial results go through the
    merge), every row of three unsplit tiles (first, middle, last), a strided sample of all rows (every 61st token)
    and 24 decode rows (longest, shortest, random); every page the append touched, bit for bit; and a finiteness
    check of every output row (a read of a NaN-poisoned page would show)."""
    w = make_workload(5)
    st = _run(w, fused=True)
    sched = R.schedule(w)
    rng = np.random.default_rng(105)
    T = sched["num_tokens"]
    for l in range(len(w.layers)):
        out = st.layers[l].out
        assert bool(torch_gpu.isfinite(out.float()).all()), "non-finite output somewhere"
        plan = st.layers[l].plan
        split_rows, n_split = _tile_rows(plan, sched["query_start_loc"], True)
        plain_rows, _ = _tile_rows(plan, sched["query_start_loc"], False, limit=3)
        toks = set(split_rows) | set(plain_rows) | set(range(0, T, 61))
        toks |= set(_sample_tokens(sched, rng, n_dec=22, per_chunk=0))
        mx, mean = H.compare(w, st, l, sorted(toks), label=f"w5 full layer {l}")
        print(f"  layer {l}: {len(toks)} rows ({n_split} split tiles, {len(split_rows)} of their rows), "
              f"max {mx:.3g} mean {mean:.3g}", flush=True)
        touched = sorted(set((sched["layers"][l]["slot_mapping"] // w.page_size).tolist()))
        _check_pages(w, st, l, touched)


def test_workload_1_matches_explicit_mask(torch_gpu):
    """The tiny A/B/C step against dense attention under the explicit (T,T) block-diagonal mask."""
    w = make_workload(1)
    st = _run(w)
    sched = R.schedule(w)
    q, k, v = R.step_inputs(w, 0, sched)
    ref = A.masked_attention(q, k, v, A.block_diagonal_causal_mask(sched["query_start_loc"]), w.scale)
    got = H.gpu_rows(st, 0, range(sched["num_tokens"]))
    assert np.abs(got - ref).max() <= H.TOL_F32_MAX


EDGE = {
    "decode ctx0 and page boundaries P16": dict(reqs=[(WAITING, 0, 1), (DECODING, 16, 1), (DECODING, 15, 1),
                                                      (DECODING, 31, 1), (DECODING, 32, 1), (DECODING, 1, 1)]),
    "page 8": dict(reqs=[(DECODING, 100, 1), (PREFILLING, 37, 45), (WAITING, 0, 70)], P=8),
    "page 64": dict(reqs=[(DECODING, 300, 1), (PREFILLING, 100, 90), (WAITING, 0, 129)], P=64),
    "page 256": dict(reqs=[(DECODING, 700, 1), (PREFILLING, 300, 300), (WAITING, 0, 257)], P=256),
    "head dim 64": dict(reqs=[(DECODING, 900, 1), (PREFILLING, 200, 150), (WAITING, 0, 65)], D=64),
    "group 16 (decode fast path limit)": dict(reqs=[(DECODING, 500, 1), (PREFILLING, 64, 20)], Hq=32, Hkv=2),
    "group 32 (decode via per-token kernel)": dict(reqs=[(DECODING, 500, 1), (PREFILLING, 64, 20)], Hq=32, Hkv=1),
    "MHA group 1": dict(reqs=[(DECODING, 333, 1), (WAITING, 0, 200)], Hq=4, Hkv=4),
    "group 8 (16 or 32 tokens per prefill tile)": dict(reqs=[(DECODING, 700, 1), (PREFILLING, 300, 100),
                                                              (WAITING, 0, 77)], Hq=16, Hkv=2),
    "bf16 page 4 (per-token kernel)": dict(reqs=[(DECODING, 77, 1), (PREFILLING, 10, 30)], P=4),
    "sliding window 0": dict(reqs=[(DECODING, 50, 1), (PREFILLING, 40, 33)], window_left=0, ring_len=8, budget=64),
    "sliding window 1": dict(reqs=[(DECODING, 50, 1), (PREFILLING, 40, 33)], window_left=1, ring_len=8, budget=64),
    "sliding window 100 P16": dict(reqs=[(DECODING, 1000, 1), (PREFILLING, 500, 200), (WAITING, 0, 150)],
                                   window_left=100, ring_len=24, budget=256),
    "fp32 long rows with splits": dict(reqs=[(DECODING, 2000, 1), (PREFILLING, 500, 60), (WAITING, 0, 40)],
                                       dtype="f32", Hq=4, Hkv=2, D=64, P=16),
    "many splits": dict(reqs=[(DECODING, 3000, 1), (DECODING, 70, 1), (PREFILLING, 1000, 300)],
                        decode_split=64, prefill_split=64),
    # fixed splits far above the page ids the kernels stage per split: capped at 1038 (decode) and 1534 (prefill)
    # pages, so the 9001-key decode row and the chunk's 12.5k-key tiles each take two splits of the largest size
    "page 8 at the page-id staging limits": dict(reqs=[(DECODING, 9000, 1), (PREFILLING, 12500, 40)], P=8,
                                                 decode_split=1 << 16, prefill_split=1 << 20),
    # decode splits of 2560 keys or more run the decode kernel with one tile in flight per wave: at the threshold,
    # rows ending just below and at a split boundary, a short row, and head dim 64
    "decode splits at the one-tile threshold": dict(reqs=[(DECODING, 6000, 1), (DECODING, 2559, 1),
                                                          (DECODING, 2560, 1), (DECODING, 33, 1),
                                                          (PREFILLING, 200, 50)], decode_split=2560),
    "head dim 64 with long decode splits": dict(reqs=[(DECODING, 5000, 1), (DECODING, 100, 1), (WAITING, 0, 40)],
                                                D=64, decode_split=4096),
    # the kernels' XCD mapping of (item, kv head) pairs: 16 kv heads (two per XCD) and 3 (no XCD grouping)
    "16 kv heads": dict(reqs=[(DECODING, 2000, 1), (DECODING, 300, 1), (PREFILLING, 500, 200), (WAITING, 0, 90)],
                        Hq=32, Hkv=16),
    "3 kv heads": dict(reqs=[(DECODING, 2000, 1), (DECODING, 300, 1), (PREFILLING, 500, 200), (WAITING, 0, 90)],
                       Hq=12, Hkv=3),
}


@pytest.mark.parametrize("fused,rows", [(False, 0), (True, 0), (True, 256)])
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(torch_gpu, name, fused, rows):
    """Each edge case with the append as its own launch and fused, and fused with 256-row prefill tiles."""
    cfg = dict(EDGE[name])
    reqs = cfg.pop("reqs")
    ds = cfg.pop("decode_split", 0)
    ps = cfg.pop("prefill_split", 0)
    w = H.custom_workload(reqs, name=name, **cfg)
    st = _run(w, fused=fused, decode_split=ds, prefill_split=ps, prefill_rows=rows)
    print(f"  plan {st.layers[0].plan.counts()}", flush=True)
    H.compare(w, st, 0, label=name)
    _check_pages(w, st, 0)


def test_long_context(torch_gpu):
    """Four times the longest context of the benchmark's workloads: a 131001-key decode row (an 8188-entry block-table
    row) and a 32-token chunk at context 100000, with the planner's splits and the fused append; every row and page
    (the index arithmetic at these sizes is what is under test, so one launch configuration suffices)."""
    w = H.custom_workload([(DECODING, 131000, 1), (PREFILLING, 100000, 32)], name="long context")
    st = _run(w, fused=True)
    print(f"  plan {st.layers[0].plan.counts()}", flush=True)
    H.compare(w, st, 0, label="long context")
    _check_pages(w, st, 0)


def test_zero_length_rows_through_the_abi(torch_gpu):
    """Rows with q_len 0 produce nothing; their neighbours are unaffected (metadata built by hand, not scheduled)."""
    import torch
    import paged_kv_attention_varlen_amd as cb
    rng = np.random.default_rng(5)
    P, Hq, Hkv, D, n_pages = 16, 8, 2, 128, 40
    qsl = np.array([0, 1, 1, 4, 4], np.int32)
    seq = np.array([20, 9, 35, 1], np.int32)
    width = 3
    table = rng.permutation(np.arange(2, n_pages))[:4 * width].reshape(4, width).astype(np.int32)
    kc = np.full((n_pages, P, Hkv, D), np.nan, np.float32)
    vc = np.full((n_pages, P, Hkv, D), np.nan, np.float32)
    from synth import round_to_bf16
    for r in range(4):
        for pos in range(int(seq[r])):
            s = A.slot_of(table[r], pos, P)
            kc[s // P, s % P] = round_to_bf16(rng.standard_normal((Hkv, D)).astype(np.float32))
            vc[s // P, s % P] = round_to_bf16(rng.standard_normal((Hkv, D)).astype(np.float32))
    q = round_to_bf16(rng.standard_normal((4, Hq, D)).astype(np.float32))
    ref = A.paged_attention(q, kc.astype(np.float64), vc.astype(np.float64), qsl, seq, table, P, 0.1)
    dev = "cuda"
    kd = torch.from_numpy(kc.transpose(0, 2, 1, 3).copy()).to(torch.bfloat16).to(dev)
    vd = torch.from_numpy(vc.transpose(0, 2, 3, 1).copy()).to(torch.bfloat16).to(dev)
    qd = torch.from_numpy(q).to(torch.bfloat16).to(dev)
    out = torch.full_like(qd, float("nan"))
    plan = cb.plan_attention(qsl, seq, None, Hq, Hkv, D, P, "bf16", -1, 64, 64)
    pd = torch.from_numpy(plan.buffer).to(dev)
    ws = torch.empty(max(1, cb.workspace_size(plan)), dtype=torch.uint8, device=dev)
    cb.paged_attention(out, qd, kd, vd, torch.from_numpy(table).to(dev), plan, pd, 0.1, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.abs(got - ref).max() <= H.TOL_BF16_MAX


def test_deterministic_and_batch_invariant(torch_gpu):
    """Same inputs twice: identical bits. With fixed split sizes, a request's rows do not depend on its batch."""
    reqs = [(DECODING, 1500, 1), (DECODING, 700, 1), (PREFILLING, 300, 100), (WAITING, 0, 90)]
    w = H.custom_workload(reqs, name="batch")
    a = _run(w, decode_split=256, prefill_split=512)
    b = _run(w, decode_split=256, prefill_split=512)
    assert torch_gpu.equal(a.layers[0].out, b.layers[0].out)
    alone = H.custom_workload(reqs[:1], name="alone", n_pages=w.layers[0].num_pages - 2)
    alone.requests[0].pages = [w.requests[0].pages[0]]
    c = _run(alone, decode_split=256, prefill_split=512)
    assert torch_gpu.equal(a.layers[0].out[0], c.layers[0].out[0])


def test_prefill_first_step(torch_gpu):
    """A step scheduled with the PrefillFirst policy (prefill work takes the budget first): every row and page against
    the oracle, which schedules with the same policy."""
    import dataclasses
    for idx in (3, 5):
        w = dataclasses.replace(make_workload(idx, mini=True), policy="prefill_first")
        st = _run(w)
        for l in range(len(w.layers)):
            H.compare(w, st, l, label=f"prefill-first w{idx} layer {l}")
            _check_pages(w, st, l)


PIPELINE_MODES = ["copy stream", "copy on compute stream", "concurrent prefill", "graph replay",
                  "graph replay, 256-row prefill tiles", "separate append", "per-phase launches with events"]


@pytest.mark.parametrize("mode", PIPELINE_MODES)
def test_pipeline_steps_match_oracle(torch_gpu, mode):
    """The benchmark's loop: steps prepared into alternating pinned/device buffers, launched with the lean path,
    repeated; every repetition of the (unchanged) step must produce the oracle's rows, and the caches the oracle's
    pages. The append is fused into cb_paged_attention except with concurrent prefill and in the separate-append
    mode; the per-phase mode launches each kernel of the step on its own call, between timing events, as the
    benchmark does for its sampled steps."""
    from harness import build_step, pipeline_for
    for idx in (3, 5):
        w = make_workload(idx, mini=True)
        st = build_step(w)
        graphs = mode.startswith("graph replay")
        pipe = pipeline_for(w, st, copy_stream=(mode != "copy on compute stream"),
                            concurrent=(mode == "concurrent prefill"), graphs=graphs,
                            fused_append=(mode != "separate append"), prefill_rows=(256 if "256" in mode else 0))
        events = None
        if mode == "per-phase launches with events":   # the benchmark's timing events (no system-scope fence)
            from paged_kv_attention_varlen_amd.hip_events import HipEvent
            events = [[HipEvent(timing=True, system_fence=False) for _ in range(6)] for _ in w.layers]
        print(f"[gpu] pipeline {mode} workload {idx} fused={pipe.fused}", flush=True)
        # every repetition is checked; graph replays (from the third step on) alternate with eager work on the
        # same stream and host synchronisations
        for rep in range(5):
            for l in range(len(w.layers)):
                st.layers[l].out.fill_(float("nan"))
            pipe.run(events)
            torch_gpu.cuda.synchronize()
            for l in range(len(w.layers)):
                H.compare(w, st, l, label=f"pipeline {mode} w{idx} layer {l} repetition {rep}")
        for l in range(len(w.layers)):
            _check_pages(w, st, l)
        if graphs:
            assert pipe.captures == 2 and pipe.replays == 5, "one graph per metadata buffer of the padded shape"
        if events is not None:
            # the events were recorded by the first and last kernels of the decode, prefill and merge calls of the
            # last step (or on the stream, for a call with nothing to launch): in stream order, and a call that ran
            # kernels took time
            for l in range(len(w.layers)):
                ev = events[l]
                for k in range(5):
                    assert ev[k].elapsed_time(ev[k + 1]) >= 0.0, (l, k)
                c = st.layers[l].plan.counts()
                for (a, b), n in (((0, 1), c["decode"]), ((2, 3), c["prefill"] + c["rowwise"]),
                                  ((4, 5), c["combine"])):
                    if n > 0:
                        assert ev[a].elapsed_time(ev[b]) > 0.0, (l, a, n)


def _append_slots(rng, P, n_pages, T):
    """Slot patterns the append kernel treats differently: aligned whole-page runs, a run that starts mid-page and
    crosses into the next page, a run broken by a skipped token, and scattered single slots; T is not a multiple of
    the kernel's 16-token groups. Every slot is used at most once."""
    c = int(rng.integers(0, n_pages - 1))                      # the crossing run uses pages c and c + 1
    pages = [int(x) for x in rng.permutation(n_pages) if x not in (c, c + 1)]
    slots = []
    for k in range(2):                                         # whole pages, in order
        slots += [pages[k] * P + o for o in range(P)][:32]
    start = c * P + max(0, P - 5)
    slots += [start + i for i in range(min(9, 2 * P - max(0, P - 5)))]
    run = [pages[2] * P + o for o in range(min(P, 16))]        # a run with one token skipped
    run[len(run) // 2] = -1
    slots += run
    free = [p_ * P + o for p_ in pages[3:] for o in range(P)]
    rng.shuffle(free)
    slots += free[:max(0, T - len(slots))]
    return np.array(slots[:T], np.int32)


@pytest.mark.parametrize("dtype,P", [("bf16", 16), ("bf16", 8), ("bf16", 32), ("bf16", 2), ("f32", 4), ("f32", 16)])
def test_kv_append_slot_patterns(torch_gpu, dtype, P):
    """cb_kv_append against the oracle's append, bit for bit, on hand-made slot patterns (whole-page runs, runs
    crossing pages, skipped tokens, scattered slots); slots never written keep their NaN."""
    import paged_kv_attention_varlen_amd as cb
    torch = torch_gpu
    rng = np.random.default_rng(11 + P)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    T = 93
    n_pages, Hkv, D = max(40, 4 * T // P), 2, (128 if dtype == "bf16" else 64)
    slots = _append_slots(rng, P, n_pages, T)
    print(f"[gpu] append {dtype} P={P} T={T}", flush=True)
    kc = torch.full((n_pages, Hkv, P, D), float("nan"), device="cuda").to(tdt)
    vc = torch.full((n_pages, Hkv, D, P), float("nan"), device="cuda").to(tdt)
    kn = torch.randn((T, Hkv, D), device="cuda").to(tdt)
    vn = torch.randn((T, Hkv, D), device="cuda").to(tdt)
    cb.kv_append(kc, vc, kn, vn, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    k_ref = np.full((n_pages, P, Hkv, D), np.nan, np.float32)
    v_ref = np.full((n_pages, P, Hkv, D), np.nan, np.float32)
    A.kv_append(k_ref, v_ref, kn.float().cpu().numpy(), vn.float().cpu().numpy(), slots, P)
    assert H.same_bits(kc.float().cpu().numpy().transpose(0, 2, 1, 3), k_ref), "K cache differs"
    assert H.same_bits(vc.float().cpu().numpy().transpose(0, 3, 1, 2), v_ref), "V cache differs"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_pages_bit_exact(torch_gpu, dtype):
    """cb_kv_copy_pages against the oracle's page copy: random page lists (some out of range, skipped), both
    directions (cache -> swap buffer with a source list, swap buffer -> cache with a destination list)."""
    import paged_kv_attention_varlen_amd as cb
    torch = torch_gpu
    rng = np.random.default_rng(3)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n_pages, n_swap = 40, 12
    for shape in ((8, 16, 128), (8, 128, 16), (2, 4, 64)):           # K page, V^T page, a small page
        cache = torch.randn((n_pages,) + shape, device="cuda").to(tdt)
        swap = torch.full((n_swap,) + shape, float("nan"), device="cuda").to(tdt)
        src = rng.permutation(n_pages)[:n_swap].astype(np.int32)
        src[3] = n_pages + 5                                           # out of range: skipped
        cb.copy_pages(swap, cache, None, torch.from_numpy(src).cuda())
        ref = np.full((n_swap,) + shape, np.nan, np.float32)
        A.copy_pages(ref, None, cache.float().cpu().numpy(), src)
        torch.cuda.synchronize()
        assert H.same_bits(swap.float().cpu().numpy(), ref)
        dst = rng.permutation(n_pages)[:n_swap].astype(np.int32)
        dst[0] = -1                                                    # skipped
        before = cache.float().cpu().numpy()
        cb.copy_pages(cache, swap, torch.from_numpy(dst).cuda(), None)
        ref = before.copy()
        A.copy_pages(ref, dst, swap.float().cpu().numpy(), None)
        torch.cuda.synchronize()
        assert H.same_bits(cache.float().cpu().numpy(), ref)


def test_swap_out_and_back_preserves_outputs(torch_gpu):
    """Offloading round trip through pinned host memory: a request's pages go out, the freed pages are poisoned,
    the request comes back into other free pages with its block-table row updated, and the step's attention output
    is bitwise what it was."""
    import torch
    from paged_kv_attention_varlen_amd.swap import HostSwap
    w = make_workload(3, mini=True)
    st = _run(w)
    L = st.layers[0]
    before = L.out.clone()
    sched = st.sched
    P = w.page_size
    used = sched["layers"][0]["used_pages"]
    spare = list(np.asarray(w.layers[0].free_pages[used:], np.int32))   # pages no row of the step holds
    for r in (0, sched["num_reqs"] - 2):                               # a decode row and a prefill row
        n = -(-int(sched["seq_lens"][r]) // P)
        old = L.block_table[r, :n].clone()
        assert len(spare) >= n, "workload pool has no spare pages for the test"
        new = torch.from_numpy(np.array([spare.pop() for _ in range(n)], np.int32)).cuda()
        pool = HostSwap(L.k_cache, L.v_cache, capacity=n)
        pool.swap_out(L.k_cache, L.v_cache, old)
        torch.cuda.synchronize()
        L.k_cache[old.long()] = float("nan")
        L.v_cache[old.long()] = float("nan")
        pool.swap_in(L.k_cache, L.v_cache, new)
        L.block_table[r, :n] = new
        L.out.fill_(float("nan"))
        st.attend(0)
        torch.cuda.synchronize()
        print(f"[gpu] swap round trip of row {r}: {n} pages", flush=True)
        assert torch.equal(L.out, before)


def test_prefix_sharing_step(torch_gpu):
    """Prefix sharing at admission, end to end. Step 1 (host only): A's 100-token prompt is admitted; its six full
    blocks are then registered in the prefix cache. Step 2: A decodes while B, whose prompt starts with A's first 96
    tokens, is admitted: the scheduler matches A's six pages, B's context starts at 96 and it prefills only its 40
    remaining tokens. The metadata (block table with the shared pages, slots) comes from cb_build_metadata and
    equals the oracle scheduler's; the device step's outputs match the oracle's paged attention over the same
    caches; and B's rows are bitwise those of a run where B holds private copies of the prefix pages."""
    import torch
    import paged_kv_attention_varlen_amd as cb
    from oracle import prefix_cache as O
    from oracle import scheduler as OS
    from synth import round_to_bf16
    rng = np.random.default_rng(21)
    P, Hq, Hkv, D, n_pages = 16, 8, 2, 128, 64
    prompt_a = rng.integers(0, 30000, 100).astype(np.int32)
    prompt_b = np.concatenate([prompt_a[:96], rng.integers(0, 30000, 40).astype(np.int32)])
    free0 = np.arange(2, n_pages, dtype=np.int32)
    pc, oc = cb.PrefixCache(n_pages, free0), O.PrefixCache(n_pages, free0.tolist())
    pools = [{"ring_len": 0, "window_left": -1, "pool_pages": n_pages - 2, "free_pages": np.zeros(0, np.int32)}]
    hashes = {0: O.block_hashes(prompt_a, P), 1: O.block_hashes(prompt_b, P)}
    assert cb.block_hashes(prompt_b, P).tolist() == hashes[1]

    def schedule(reqs):
        hs = [hashes[r.id] for r in reqs]
        got = cb.build_metadata(reqs, pools, 512, 8, P, 0.0, 0, prefix_cache=pc, prompt_hashes=hs)
        want = OS.build_metadata(reqs, pools, 512, 8, P, 0.0, 0, prefix_cache=oc, prompt_hashes=hs)
        for key in ("query_start_loc", "seq_lens", "matched_tokens"):
            assert np.array_equal(got[key], want[key]), key
        for key in ("block_table", "slot_mapping"):
            assert np.array_equal(got["layers"][0][key], want["layers"][0][key]), key
        return got, hs

    reqs = [cb.Request(0, WAITING, 0, 100, [np.zeros(0, np.int32)])]
    s1, hs = schedule(reqs)
    reqs, _ = cb.advance(reqs, s1, [np.zeros(0, np.int32)], [0], P, pc, hs)
    OS.advance([cb.Request(0, WAITING, 0, 100, [np.zeros(0, np.int32)])], s1, [np.zeros(0, np.int32)], P, oc, hs)
    pages_a = reqs[0].pages[0]
    assert pc.stats()[2] == 6                                            # A's six full blocks are registered
    reqs.append(cb.Request(1, WAITING, 0, len(prompt_b), [np.zeros(0, np.int32)]))
    s2, _ = schedule(reqs)
    qsl, seq = s2["query_start_loc"], s2["seq_lens"]
    table, slots = s2["layers"][0]["block_table"], s2["layers"][0]["slot_mapping"]
    assert s2["matched_tokens"].tolist() == [0, 96] and seq.tolist() == [101, 136]
    assert table[1, :6].tolist() == pages_a[:6].tolist()                 # B's first six pages are A's
    assert pc.page_info(int(pages_a[0]))[0] == 2

    # caches: A's history (100 keys) on its pages; B's context is A's (same tokens, same pages)
    kc = np.full((n_pages, P, Hkv, D), np.nan, np.float32)
    vc = np.full((n_pages, P, Hkv, D), np.nan, np.float32)
    hist_k = round_to_bf16(rng.standard_normal((100, Hkv, D)).astype(np.float32))
    hist_v = round_to_bf16(rng.standard_normal((100, Hkv, D)).astype(np.float32))
    for pos in range(100):
        kc[pages_a[pos // P], pos % P] = hist_k[pos]
        vc[pages_a[pos // P], pos % P] = hist_v[pos]
    T = int(qsl[-1])
    new_k = round_to_bf16(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    new_v = round_to_bf16(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    q = round_to_bf16(rng.standard_normal((T, Hq, D)).astype(np.float32))

    def run(tab, sl, kcache, vcache):
        kd = torch.from_numpy(kcache.transpose(0, 2, 1, 3).copy()).to(torch.bfloat16).cuda()
        vd = torch.from_numpy(vcache.transpose(0, 2, 3, 1).copy()).to(torch.bfloat16).cuda()
        cb.kv_append(kd, vd, torch.from_numpy(new_k).to(torch.bfloat16).cuda(),
                     torch.from_numpy(new_v).to(torch.bfloat16).cuda(), torch.from_numpy(sl).cuda())
        qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
        out = torch.full_like(qd, float("nan"))
        plan = cb.plan_attention(qsl, seq, None, Hq, Hkv, D, P, "bf16", -1, 0, 0)
        pd = torch.from_numpy(plan.buffer).cuda()
        ws = torch.empty(max(1, cb.workspace_size(plan)), dtype=torch.uint8, device="cuda")
        cb.paged_attention(out, qd, kd, vd, torch.from_numpy(tab).cuda(), plan, pd, 1 / np.sqrt(D), ws)
        torch.cuda.synchronize()
        return out

    got = run(table, slots, kc, vc)
    ko, vo = kc.copy(), vc.copy()
    A.kv_append(ko, vo, new_k, new_v, slots, P)
    ref = A.paged_attention(q, ko.astype(np.float64), vo.astype(np.float64), qsl, seq, table, P, 1 / np.sqrt(D))
    err = np.abs(got.float().cpu().numpy() - ref)
    assert err.max() <= H.TOL_BF16_MAX and err.mean() <= H.TOL_BF16_MEAN
    # without sharing: B's prefix copied to private pages; B's rows are bitwise the same
    spare = [p for p in range(2, n_pages) if p not in set(table.reshape(-1).tolist())][:6]
    private = table.copy()
    private[1, :6] = spare
    kp, vp = kc.copy(), vc.copy()
    kp[spare], vp[spare] = kc[pages_a[:6]], vc[pages_a[:6]]
    sl_private = np.array([private[r][p // P] * P + p % P for r, p in
                           [(0, 100)] + [(1, x) for x in range(96, 136)]], np.int32)
    alone = run(private, sl_private, kp, vp)
    assert torch.equal(got[1:], alone[1:])
