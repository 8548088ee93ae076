"""cb_paged_attention_noalloc (the entry point for callers that cannot allocate) against cb_paged_attention with a
caller workspace: two calls in a row through the C ABI, the second on a smaller step, each bitwise equal to the
workspace entry point's output on the same inputs (same plans, same kernels; only the scratch memory differs)."""
import ctypes as C

import numpy as np
import pytest

from synth import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_varlen_amd import load_library
    load_library()
    return torch


def _args(L, scale):
    import paged_kv_attention_varlen_amd as cb
    return cb._args(L.out, L.q, L.k_cache, L.v_cache, L.block_table, L.plan, L.plan_dev, scale, L.workspace)


def test_noalloc_matches_workspace_entry_point(torch_gpu):
    torch = torch_gpu
    from harness import build_step
    from paged_kv_attention_varlen_amd import _abi
    lib = _abi.load()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    # first the full mixed 2048-token step (21 MiB of split partials), then a reduced hybrid pair (smaller)
    for idx, mini in ((3, False), (5, True)):
        w = make_workload(idx, mini=mini)
        print(f"[gpu] noalloc vs workspace: {w.name}", flush=True)
        st = build_step(w)
        for l, L in enumerate(st.layers):
            assert cb_workspace(L) <= _abi.CB_NOALLOC_WORKSPACE_BYTES
        st.run(fused_append=False)                    # append + attention with the caller's workspace
        torch.cuda.synchronize()
        ref = [L.out.clone() for L in st.layers]
        for l, L in enumerate(st.layers):
            L.out.fill_(float("nan"))
            a = _args(L, st.scale)
            a.workspace, a.workspace_bytes = None, 0   # ignored by the allocation-free entry point
            assert lib.cb_paged_attention_noalloc(C.byref(a), stream) == _abi.CB_OK
        torch.cuda.synchronize()
        for l, L in enumerate(st.layers):
            assert bool(torch.isfinite(L.out.float()).all())
            assert torch.equal(L.out, ref[l]), f"{w.name} layer {l}: outputs differ"


def cb_workspace(L):
    import paged_kv_attention_varlen_amd as cb
    return cb.workspace_size(L.plan)


def test_noalloc_refuses_a_plan_beyond_its_array(torch_gpu):
    from paged_kv_attention_varlen_amd import _abi
    lib = _abi.load()
    a = _abi.cb_attn_args()
    a.layout = _abi.CB_LAYOUT_KD_VT
    a.shape = _abi.cb_attn_shape(32, 8, 128, 16, 1, -1, 0, 0)
    a.plan_info.n_decode = 1
    a.plan_info.n_partials = (_abi.CB_NOALLOC_WORKSPACE_BYTES // (32 * 128 * 4)) + 1
    assert lib.cb_paged_attention_noalloc(C.byref(a), None) == _abi.CB_E_WORKSPACE
