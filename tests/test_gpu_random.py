"""GPU parity on random small steps: random request mixes (decodes, continuing chunks, new prompts), page sizes,
head dims, head groups, sliding windows, split sizes, prefill tile sizes and append modes, each compared with the
fp64 oracle on every output row and every cache page. Tolerances as in test_gpu_parity."""
import numpy as np
import pytest

from oracle import reference as R
from synth import DECODING, PREFILLING, WAITING
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


def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    P = int(rng.choice([8, 16, 32, 64]))
    D = int(rng.choice([64, 128]))
    Hq, Hkv = [(8, 2), (32, 8), (4, 4), (16, 1), (32, 2)][int(rng.integers(5))]
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    budget = int(rng.choice([256, 1024, 2048]))
    reqs = []
    for _ in range(int(rng.integers(1, 13))):
        kind = rng.choice(["decode", "chunk", "new"])
        if kind == "decode":
            reqs.append((DECODING, int(rng.integers(1, 3000)), 1))
        elif kind == "chunk":
            reqs.append((PREFILLING, int(rng.integers(1, 2000)), int(rng.integers(2, 400))))
        else:
            reqs.append((WAITING, 0, int(rng.integers(1, 500))))
    cfg = dict(Hq=Hq, Hkv=Hkv, D=D, P=P, dtype=dtype, budget=budget, seed=int(seed))
    if rng.random() < 0.35:
        W = int(rng.choice([0, 1, 37, 300, 1500]))
        # the ring must hold the window plus the step's chunk: (W + chunk + P - 2) / P + 1 pages
        cfg.update(window_left=W, ring_len=(W + budget + P - 2) // P + 2)
    run = dict(decode_split=int(rng.choice([0, 64, 256])), prefill_split=int(rng.choice([0, 64, 512])),
               prefill_rows=int(rng.choice([0, 128, 256])))
    fused = bool(rng.random() < 0.5)
    return reqs, cfg, run, fused


@pytest.mark.parametrize("seed", range(48))
def test_random_step_matches_oracle(torch_gpu, seed):
    from harness import build_step
    reqs, cfg, run, fused = _random_case(seed)
    w = H.custom_workload(reqs, name=f"random {seed}", **cfg)
    print(f"[gpu] random {seed}: {len(reqs)} requests {cfg} {run} fused={fused}", flush=True)
    st = build_step(w, **run)
    st.run(fused_append=fused)
    torch_gpu.cuda.synchronize()
    print(f"  plan {st.layers[0].plan.counts()}", flush=True)
    H.compare(w, st, 0, label=f"random {seed}")
    ids, k_ref, v_ref = R.pages_reference(w, 0, R.schedule(w), None)
    k, v = H.logical_cache(st, 0)
    assert H.same_bits(k[ids], k_ref), "K cache differs"
    assert H.same_bits(v[ids], v_ref), "V cache differs"
