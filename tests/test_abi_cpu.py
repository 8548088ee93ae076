"""The C-ABI library loads, exports every symbol include/cb.h declares, and the ctypes mirror matches the C layout.
No compute runs on a device here."""
import os
import re
import subprocess
import tempfile

import pytest

from paged_kv_attention_varlen_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cb.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(cb_[a-z_0-9]+)\s*\(", text, re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _abi.load()
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (cb_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings():
    lib = _abi.load()
    assert lib.cb_abi_version() == _abi.ABI_VERSION
    for st in range(7):
        assert lib.cb_status_str(st)
    assert lib.cb_status_str(99) == b"unknown status"


STRUCTS = ["cb_req", "cb_layer_pool", "cb_sched_params", "cb_step", "cb_attn_shape", "cb_plan", "cb_attn_args"]


def test_ctypes_layout_matches_c():
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "cb.h"', "int main(void){"]
    for s in STRUCTS:
        src.append(f'printf("{s} %zu\\n", sizeof({s}));')
        for f, _ in getattr(_abi, s)._fields_:
            src.append(f'printf("{s}.{f} %zu\\n", offsetof({s}, {f}));')
    src.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write("\n".join(src))
        exe = os.path.join(d, "layout")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = dict(zip(lines[0::2], map(int, lines[1::2])))
    import ctypes
    for s in STRUCTS:
        cls = getattr(_abi, s)
        assert ctypes.sizeof(cls) == got[s], s
        for f, _ in cls._fields_:
            assert getattr(cls, f).offset == got[f"{s}.{f}"], (s, f)


def test_device_calls_reject_bad_arguments_without_launching():
    import ctypes as C
    lib = _abi.load()
    # invalid sizes are refused before any HIP call
    KDVT = _abi.CB_LAYOUT_KD_VT
    assert lib.cb_kv_append(None, None, None, None, None, -1, 1, 16, 8, 128, 1, KDVT, None) == _abi.CB_E_INVAL
    assert lib.cb_kv_append(None, None, None, None, None, 4, 1, 16, 8, 128, 7, KDVT, None) == _abi.CB_E_UNSUPPORTED
    assert lib.cb_kv_append(None, None, None, None, None, 0, 1, 16, 8, 128, 1, KDVT, None) == _abi.CB_OK
    # the plain [page][offset][head][d] layout tag (and any unknown tag) is refused before any launch
    for tag in (_abi.CB_LAYOUT_PAGED_NHD, 7):
        assert lib.cb_kv_append(None, None, None, None, None, 4, 1, 16, 8, 128, 1, tag, None) == _abi.CB_E_UNSUPPORTED
    a = _abi.cb_attn_args()
    a.shape = _abi.cb_attn_shape(32, 8, 128, 16, 1, -1, 0, 0)
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_UNSUPPORTED   # zeroed args: layout tag 0
    a.layout = 5
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_UNSUPPORTED
    a.layout = KDVT
    a.shape = _abi.cb_attn_shape(32, 8, 96, 16, 1, -1, 0, 0)
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_UNSUPPORTED
    a.shape = _abi.cb_attn_shape(32, 8, 128, 16, 1, -1, 0, 0)
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_OK          # empty plan: nothing to do
    a.plan_info.n_decode = 3
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_INVAL     # null pointers
    a.phases = 99
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_INVAL
    # fused append: k_new without v_new / slot_mapping, or a token count other than the plan's, is refused before
    # any launch (the pointers below are never dereferenced)
    a.phases = 0
    a.out = a.q = a.k_cache = a.v_cache = a.block_table = a.plan = 4096
    a.num_pages, a.table_width = 8, 4
    a.plan_info.num_tokens = 3
    a.k_new = 4096
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_INVAL
    a.v_new = a.slot_mapping = 4096
    a.num_new = 2
    assert lib.cb_paged_attention(C.byref(a), None) == _abi.CB_E_INVAL
    # page copies: sizes checked before any launch
    assert lib.cb_kv_copy_pages(None, None, 4, None, None, 4, 0, 4096, None) == _abi.CB_OK      # nothing to copy
    assert lib.cb_kv_copy_pages(None, None, 4, None, None, 4, -1, 4096, None) == _abi.CB_E_INVAL
    assert lib.cb_kv_copy_pages(None, None, 4, None, None, 4, 2, 4100, None) == _abi.CB_E_INVAL  # not 16-aligned
    assert lib.cb_kv_copy_pages(None, None, 4, None, None, 4, 2, 4096, None) == _abi.CB_E_INVAL  # null buffers
    assert lib.cb_kv_copy_pages(1, None, 4, 1, None, 8, 6, 4096, None) == _abi.CB_E_INVAL        # 6 pages > 4 slots
    assert lib.cb_kv_copy_pages(1, None, 8, 1, None, 8, 2, 1 << 40, None) == _abi.CB_E_UNSUPPORTED


def test_slot_mapping_follows_the_table_rule():
    """cb_slot_mapping: page * P + offset of each position, through the block-table row or the ring; refuses
    positions whose table entry does not exist."""
    import numpy as np
    import paged_kv_attention_varlen_amd as cb
    pages = np.array([7, 18, 3], np.int32)
    # the blog's worked example: request C on pages [7, 18] with BLOCK_SIZE 2: positions 0..2 -> 14, 15, 36
    assert cb.slot_mapping(pages[:2], 0, 2, 0, 3).tolist() == [14, 15, 36]
    assert cb.slot_mapping(pages, 0, 4, 5, 12).tolist() == [18 * 4 + 1, 18 * 4 + 2, 18 * 4 + 3, 12, 13, 14, 15]
    # ring of 2 pages: logical page 2 reuses ring slot 0
    assert cb.slot_mapping(pages[:2], 2, 2, 3, 6).tolist() == [37, 14, 15]
    assert cb.slot_mapping(pages, 0, 4, 3, 3).size == 0
    with pytest.raises(cb.CbError):
        cb.slot_mapping(pages[:2], 0, 2, 0, 5)          # position 4 needs a third page


def test_validate_metadata_finds_each_kind_of_corruption():
    import numpy as np
    import paged_kv_attention_varlen_amd as cb
    from synth import make_workload
    from harness import sched_pools
    w = make_workload(3, mini=True)
    pools, pad = sched_pools(w)
    s = cb.build_metadata(w.requests, pools, w.max_batch_tokens, w.max_requests, w.page_size, 0.0, pad)
    L = s["layers"][0]
    n_pages = w.layers[0].num_pages
    args = (s["query_start_loc"], s["seq_lens"], L["block_table"], None, L["slot_mapping"], n_pages, w.page_size, 2)
    assert cb.validate_metadata(*args) is None
    bt = L["block_table"].copy()
    bt[1, 0] = n_pages                                   # outside the pool
    assert cb.validate_metadata(args[0], args[1], bt, *args[3:]) == ("block_table", 1)
    bt = L["block_table"].copy()
    bt[2, 0] = 1                                         # a padding page in a used entry
    assert cb.validate_metadata(args[0], args[1], bt, *args[3:]) == ("block_table", 2)
    sm = L["slot_mapping"].copy()
    sm[5] += 1                                           # a slot off the table rule
    assert cb.validate_metadata(*args[:4], sm, *args[5:]) == ("slot_mapping", 5)
    sm[5] = -1                                           # a skipped token is fine
    assert cb.validate_metadata(*args[:4], sm, *args[5:]) is None
    qsl = s["query_start_loc"].copy()
    qsl[2] = qsl[1] - 1
    assert cb.validate_metadata(qsl, *args[1:])[0] == "query_start_loc"
    seq = s["seq_lens"].copy()
    seq[-1] = 0
    assert cb.validate_metadata(args[0], seq, *args[2:])[0] in ("seq_lens",)


def test_dtype_mismatch_raises_before_any_launch(monkeypatch):
    """The C ABI sees only pointers: the binding refuses tensors whose dtype is not the plan's before calling it."""
    import numpy as np
    import torch
    import paged_kv_attention_varlen_amd as cb

    class NoLaunch:
        def __getattr__(self, name):
            raise AssertionError(f"{name} must not be called")

    plan = cb.plan_attention(np.array([0, 1, 3], np.int32), np.array([5, 4], np.int32), None, 8, 2, 128, 16,
                             "bf16")
    monkeypatch.setattr(cb, "_check_dev", lambda t, name: None)
    monkeypatch.setattr(cb._abi, "load", lambda *a: NoLaunch())
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros((3, 8, 128), dtype=bf)
    kc = torch.zeros((4, 2, 16, 128), dtype=bf)
    vc = torch.zeros((4, 2, 128, 16), dtype=bf)
    bt = torch.zeros((2, 1), dtype=torch.int32)
    pd = torch.from_numpy(plan.buffer)
    for bad in ("q", "out", "k_cache", "v_cache"):
        t = dict(q=q, out=q.clone(), k_cache=kc, v_cache=vc)
        t[bad] = t[bad].to(f32)
        with pytest.raises(ValueError, match=bad):
            cb.paged_attention(t["out"], t["q"], t["k_cache"], t["v_cache"], bt, plan, pd, 0.1)
    with pytest.raises(ValueError, match="block_table"):
        cb.paged_attention(q.clone(), q, kc, vc, bt.to(torch.int64), plan, pd, 0.1)
    with pytest.raises(ValueError, match="k_new"):
        cb.paged_attention(q.clone(), q, kc, vc, bt, plan, pd, 0.1, k_new=torch.zeros((3, 2, 128), dtype=f32),
                           v_new=torch.zeros((3, 2, 128), dtype=bf), slot_mapping=torch.zeros(3, dtype=torch.int32))
