"""Every module of the package, the benchmark and the entry point import cleanly without a GPU."""
import importlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_package_modules_import():
    for m in ("paged_kv_attention_varlen_amd", "paged_kv_attention_varlen_amd._abi",
              "paged_kv_attention_varlen_amd.step", "paged_kv_attention_varlen_amd.build", "harness",
              "harness.device_step"):
        importlib.import_module(m)


def test_bench_and_entry_point_import():
    sys.path.insert(0, ROOT)
    try:
        bench = importlib.import_module("bench")
        assert callable(bench.main)
        entry = importlib.import_module("__graft_entry__")
        assert callable(entry.build) and callable(entry.smoke)
    finally:
        sys.path.remove(ROOT)


def test_package_holds_no_workload_code():
    """The product package neither imports the synthetic-workload modules nor the oracle."""
    pkg = os.path.join(ROOT, "paged_kv_attention_varlen_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            text = open(os.path.join(pkg, name)).read()
            for banned in ("import synth", "from synth", "import oracle", "from oracle", "import harness",
                           "from harness"):
                assert banned not in text, (name, banned)
