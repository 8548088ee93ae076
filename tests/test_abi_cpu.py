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
    assert lib.cb_kv_append(None, None, None, None, None, -1, 1, 16, 8, 128, 1, None) == _abi.CB_E_INVAL
    assert lib.cb_kv_append(None, None, None, None, None, 4, 1, 16, 8, 128, 7, None) == _abi.CB_E_UNSUPPORTED
    assert lib.cb_kv_append(None, None, None, None, None, 0, 1, 16, 8, 128, 1, None) == _abi.CB_OK
    a = _abi.cb_attn_args()
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
