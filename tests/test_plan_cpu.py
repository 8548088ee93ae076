"""cb_plan_attention: every query row's visible key range is covered exactly once by its work items, split rows have
one merge entry naming exactly their partial slots, and unsupported shapes fall back to per-token items."""
import numpy as np
import pytest

import paged_kv_attention_varlen_amd as cb


def _cover_check(qsl, seq, ring, plan, window):
    T = int(qsl[-1])
    dec, pre, row, comb = (plan.items(k) for k in ("decode", "prefill", "rowwise", "combine"))
    per_tok = {t: [] for t in range(T)}
    for it in np.concatenate([dec, row]) if len(dec) + len(row) else []:
        r, t, pos, a, b, slot, rl, _ = (int(x) for x in it)
        per_tok[t].append((a, b, slot, 1))
        assert rl == (0 if ring is None else ring[r])
    for it in pre:
        r, t0, pos0, qc, a, b, sb, rl = (int(x) for x in it)
        assert 1 <= qc <= plan.info.prefill_tokens
        for i in range(qc):
            per_tok[t0 + i].append((a, b, -1 if sb < 0 else sb + i, qc))
    merges = {int(c[0]): c for c in comb}
    slots_seen = set()
    for r in range(len(seq)):
        q = int(qsl[r + 1] - qsl[r])
        ctx = int(seq[r]) - q
        for i in range(q):
            t = int(qsl[r]) + i
            pos = ctx + i
            lo = 0 if window < 0 else max(0, pos - window)
            items = per_tok[t]
            assert items, t
            cov = np.zeros(pos + 1, dtype=int)
            for a, b, slot, _ in items:
                a2, b2 = max(a, lo), min(b, pos + 1)
                if b2 > a2:
                    cov[a2:b2] += 1
            assert (cov[lo:] == 1).all() and (cov[:lo] == 0).all(), (t, items)
            if len(items) == 1:
                assert items[0][2] == -1 and t not in merges
            else:
                m = merges[t]
                n, first, stride = int(m[2]), int(m[1]), int(m[3])
                assert n == len(items)
                want = sorted(first + s * stride for s in range(n))
                assert sorted(x[2] for x in items) == want
                assert not (set(want) & slots_seen)
                slots_seen |= set(want)
    assert all(s < plan.info.n_partials for s in slots_seen)


def _random(rng):
    N = int(rng.integers(1, 14))
    q = rng.choice([0, 1, 1, 1, 2, 5, 33, 130, 300], size=N)
    ctx = rng.integers(0, 3000, size=N)
    qsl = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    return qsl, (ctx + q).astype(np.int32)


@pytest.mark.parametrize("seed", range(40))
def test_plan_covers_every_row_exactly_once(seed):
    rng = np.random.default_rng(seed)
    qsl, seq = _random(rng)
    window = int(rng.choice([-1, -1, 0, 100, 1000]))
    ring = None if window < 0 else np.full(len(seq), 50, np.int32)
    Hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8, 32]))
    dtype = str(rng.choice(["bf16", "f32"]))
    P = int(rng.choice([2, 8, 16, 32]))
    ds = int(rng.choice([0, 64, 256]))
    ps = int(rng.choice([0, 64, 512]))
    rows = int(rng.choice([0, 128, 256]))
    plan = cb.plan_attention(qsl, seq, ring, Hkv * G, Hkv, 128, P, dtype, window, ds, ps, rows)
    _cover_check(qsl, seq, ring, plan, window)
    if plan.info.n_prefill:
        assert plan.info.prefill_tokens * G == (rows or plan.info.prefill_tokens * G)
        assert plan.info.prefill_tokens * G in (128, 256)
    c = plan.counts()
    fast = dtype == "bf16" and P >= 8
    if not fast:
        assert c["decode"] == 0 and c["prefill"] == 0
    if fast and G <= 16:
        assert c["rowwise"] == 0


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_plan_of_workloads(idx):
    from synth import make_workload
    w = make_workload(idx)
    from oracle.reference import schedule
    s = schedule(w)
    for l, lay in enumerate(w.layers):
        ring = s["layers"][l]["ring_len"] if lay.ring_len > 0 else None
        plan = cb.plan_attention(s["query_start_loc"], s["seq_lens"], ring, w.Hq, w.Hkv, w.D, w.page_size, w.dtype,
                                 lay.window_left)
        _cover_check(s["query_start_loc"], s["seq_lens"], ring, plan, lay.window_left)
        assert plan.info.max_page_index < s["layers"][l]["width"]
        if w.dtype == "f32":
            assert plan.counts()["rowwise"] >= s["num_tokens"]


def test_prefill_rows_choice():
    """256-row tiles when the chunks give at least three such work groups per CU (256 CUs), else 128; a
    requested size is honoured."""
    G, Hkv = 4, 8
    big = [0, 2048, 4096, 6144, 8064]                   # three 2048-token chunks and a 1920-token one: 126 tiles
    seq = [6144, 14336, 18432, 1920]
    plan = cb.plan_attention(big, seq, None, G * Hkv, Hkv, 128, 32, "bf16")
    assert plan.info.prefill_tokens * G == 256
    small = [0, 512, 1024]                              # 16 tiles x 8 heads: far fewer than 3 per CU
    plan = cb.plan_attention(small, [4096, 512], None, G * Hkv, Hkv, 128, 32, "bf16")
    assert plan.info.prefill_tokens * G == 128
    for rows in (128, 256):
        plan = cb.plan_attention(small, [4096, 512], None, G * Hkv, Hkv, 128, 32, "bf16", -1, 0, 0, rows)
        assert plan.info.prefill_tokens * G == rows
        _cover_check(np.array(small), np.array([4096, 512]), None, plan, -1)
    with pytest.raises(cb.CbError):
        cb.plan_attention(small, [4096, 512], None, G * Hkv, Hkv, 128, 32, "bf16", -1, 0, 0, 192)


def test_plan_rejects_bad_input():
    with pytest.raises(cb.CbError):
        cb.plan_attention([0, 2], [1], None, 8, 2, 128, 16, "bf16")          # seq_len < q_len
    with pytest.raises(cb.CbError):
        cb.plan_attention([0, 1], [5], None, 8, 3, 128, 16, "bf16")          # Hq not a multiple of Hkv
    with pytest.raises(cb.CbError):
        cb.plan_attention([0, 1], [5], None, 8, 2, 96, 16, "bf16")           # head_dim
    with pytest.raises(cb.CbError):
        cb.plan_attention([0, 1], [5], None, 8, 2, 128, 12, "bf16")          # page size
    with pytest.raises(cb.CbError):
        cb.plan_attention([0, 1], [5], None, 8, 2, 128, 16, "bf16", -1, 100)  # split not a multiple of 64
    empty = cb.plan_attention([0], [], None, 8, 2, 128, 16, "bf16")
    assert empty.info.used == 0


@pytest.mark.parametrize("P", [8, 16])
def test_split_caps_at_page_staging_limits(P):
    """A caller-fixed split is capped at the pages the kernels stage in LDS per split (decode 1038, prefill 1534;
    rounded down to a multiple of 64 keys); the cap depends on the page size only, and the rows stay covered."""
    qsl = np.array([0, 1, 41], np.int32)                       # one decode row, one 40-token chunk
    seq = np.array([9001, 12540], np.int32) * (P // 8)
    plan = cb.plan_attention(qsl, seq, None, 32, 8, 128, P, "bf16", -1, 1 << 16, 1 << 20)
    dec_cap, pre_cap = 1038 * P // 64 * 64, 1534 * P // 64 * 64
    assert plan.info.decode_split == dec_cap and plan.info.prefill_split == pre_cap
    assert plan.counts()["decode"] == -(-int(seq[0]) // dec_cap) == 2
    # each prefill tile (prefill_tokens tokens) reaches past the cap: two pieces per tile
    n_tiles = -(-40 // plan.info.prefill_tokens)
    assert plan.counts()["prefill"] == 2 * n_tiles
    _cover_check(qsl, seq, None, plan, -1)
    # below the caps a fixed split is used as given
    small = cb.plan_attention(qsl, seq, None, 32, 8, 128, P, "bf16", -1, 1024, 2048)
    assert small.info.decode_split == 1024 and small.info.prefill_split == 2048


def test_build_step_equals_build_then_plan_per_layer():
    """cb_build_step (schedule and plan every layer in one call) writes the same metadata and the same plans as
    cb_build_metadata followed by cb_plan_attention per layer, for every workload; a buffer too small for the plans
    reports CB_E_CAPACITY."""
    import ctypes as C
    import numpy as np
    import paged_kv_attention_varlen_amd as cb
    from paged_kv_attention_varlen_amd import _abi
    from harness.device_step import scheduler_for
    from synth import make_workload
    for idx in (1, 2, 3, 4, 5):
        w = make_workload(idx)
        s = scheduler_for(w)
        L = len(w.layers)
        dt = _abi.CB_DTYPE_BF16 if w.dtype == "bf16" else _abi.CB_DTYPE_F32
        shapes = [_abi.cb_attn_shape(w.Hq, w.Hkv, w.D, w.page_size, dt, lay.window_left, 0, 0, 0) for lay in w.layers]
        meta = 1 << 20
        buf = np.full(meta + (1 << 20), -7, dtype=np.int32)
        hdr, plans, offs = _abi.cb_step(), (_abi.cb_plan * L)(), (C.c_int64 * L)()
        s.build_step_into(buf.ctypes.data, meta, buf.size, (_abi.cb_attn_shape * L)(*shapes), hdr, plans, offs)
        ref = np.full(meta, -7, dtype=np.int32)
        rh = s.build_into(ref)
        assert hdr.used == rh.used and np.array_equal(buf[:rh.used], ref[:rh.used]), idx
        N = rh.num_reqs
        qsl = ref[rh.off_query_start_loc:rh.off_query_start_loc + N + 1]
        seq = ref[rh.off_seq_lens:rh.off_seq_lens + N]
        for l in range(L):
            ring = ref[rh.off_ring_len[l]:rh.off_ring_len[l] + N] if w.layers[l].ring_len > 0 else None
            want = cb.plan_into(qsl, seq, ring, shapes[l], np.zeros(1 << 20, dtype=np.int32))
            got = buf[meta + offs[l]:meta + offs[l] + plans[l].used]
            assert C.string_at(C.addressof(plans[l]), C.sizeof(_abi.cb_plan)) == \
                C.string_at(C.addressof(want.info), C.sizeof(_abi.cb_plan)), (idx, l)
            assert np.array_equal(got, want.buffer), (idx, l)
        small = np.zeros(rh.used + 16, dtype=np.int32)
        try:
            s.build_step_into(small.ctypes.data, rh.used, small.size, (_abi.cb_attn_shape * L)(*shapes), hdr, plans,
                              offs)
            raise AssertionError("expected CB_E_CAPACITY")
        except cb.CbError as e:
            assert e.status == cb.CB_E_CAPACITY
