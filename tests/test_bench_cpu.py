"""The benchmark's algorithmic work, the numerators of its rooflines, checked two ways: against a row-by-row count
over the oracle's visible key range (oracle.attention.visible_range), and against the totals the scope table
states for the workloads (prefill flops to four digits; decode bytes against the expectation of each workload's
context distribution, which a seeded draw meets only approximately)."""
import numpy as np
import pytest

import bench
from oracle import attention as A
from oracle import reference as R
from synth import make_workload


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_algorithmic_work_matches_row_by_row_count(idx):
    w = make_workload(idx)
    sched = R.schedule(w)
    work = bench.algorithmic_work(w, sched)
    qsl, seq = sched["query_start_loc"], sched["seq_lens"]
    e = 2 if w.dtype == "bf16" else 4
    for l, lay in enumerate(w.layers):
        dec_bytes = pre_flops = 0
        for r in range(sched["num_reqs"]):
            q = int(qsl[r + 1] - qsl[r])
            ctx = int(seq[r]) - q
            for i in range(q):
                lo, hi = A.visible_range(ctx + i, lay.window_left)
                n = hi - lo + 1
                if q == 1:   # K and V rows of every kv head, plus the row's Q and O
                    dec_bytes += n * w.Hkv * 2 * w.D * e + 2 * w.Hq * w.D * e
                else:        # Q.K^T and P.V: 2 flops each per (row, query head, key, d)
                    pre_flops += n * w.Hq * 4 * w.D
        assert work[l]["decode_bytes"] == dec_bytes, (idx, l)
        assert work[l]["prefill_flops"] == pre_flops, (idx, l)
        assert work[l]["append_bytes"] == 4 * int(sched["num_tokens"]) * w.Hkv * w.D * e


# totals stated for the workloads: prefill flops of the chunks (mixed step: 45.73 GFLOP; layer pair: 1.233 TFLOP
# full, 0.443 TFLOP sliding), and the decode kernel's expected K/V bytes (decode-only ~554 MB, mixed ~1.66 GB,
# large batch ~3.5 GB, layer pair ~8.66 GB full and ~2.0 GB sliding)
# (decode bytes, (prefill flops, significant digits stated))
STATED = {2: [(0.554e9, None)], 3: [(1.66e9, (45.73e9, 4))], 4: [(3.5e9, None)],
          5: [(8.66e9, (1.233e12, 4)), (2.0e9, (0.443e12, 3))]}


@pytest.mark.parametrize("idx", sorted(STATED))
def test_algorithmic_work_matches_stated_totals(idx):
    w = make_workload(idx)
    work = bench.algorithmic_work(w, R.schedule(w))
    for l, (dec, pre) in enumerate(STATED[idx]):
        # the draw's mean context differs from the distribution's by a few percent
        assert abs(work[l]["decode_bytes"] / dec - 1) < 0.07, (idx, l, work[l]["decode_bytes"])
        if pre is None:
            assert work[l]["prefill_flops"] == 0
        else:
            value, digits = pre
            # equal to the stated value when rounded to its digits
            assert abs(work[l]["prefill_flops"] / value - 1) <= 0.5 * 10 ** (1 - digits), (idx, l)
