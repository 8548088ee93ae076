"""ctypes mirror of include/cb.h and the loader of the in-tree libcb.so."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcb.so")

CB_OK, CB_E_INVAL, CB_E_NOSPACE, CB_E_CAPACITY, CB_E_UNSUPPORTED, CB_E_WORKSPACE, CB_E_HIP = range(7)
CB_DTYPE_F32, CB_DTYPE_BF16 = 0, 1
CB_DECODING, CB_PREFILLING, CB_WAITING = 0, 1, 2
CB_MAX_LAYERS = 2
CB_PHASE_DECODE, CB_PHASE_ROWWISE, CB_PHASE_PREFILL, CB_PHASE_COMBINE = 1, 2, 4, 8
CB_POLICY_FIFO, CB_POLICY_PREFILL_FIRST = 0, 1
ABI_VERSION = 8
CB_LAYOUT_PAGED_NHD, CB_LAYOUT_KD_VT = 0, 1
CB_NOALLOC_WORKSPACE_BYTES = 96 << 20

i32p = C.POINTER(C.c_int32)


class cb_req(C.Structure):
    _fields_ = [("id", C.c_int64), ("state", C.c_int32), ("num_computed", C.c_int32), ("num_pending", C.c_int32),
                ("n_pages", C.c_int32 * CB_MAX_LAYERS), ("pages", i32p * CB_MAX_LAYERS),
                ("prompt_hashes", C.POINTER(C.c_uint64)), ("n_prompt_blocks", C.c_int32)]


class cb_layer_pool(C.Structure):
    _fields_ = [("ring_len", C.c_int32), ("window_left", C.c_int32), ("pool_pages", C.c_int32),
                ("n_free", C.c_int32), ("free_pages", i32p)]


class cb_sched_params(C.Structure):
    _fields_ = [("max_batch_tokens", C.c_int32), ("max_requests", C.c_int32), ("page_size", C.c_int32),
                ("pad_page", C.c_int32), ("n_layers", C.c_int32), ("policy", C.c_int32),
                ("safety_margin", C.c_float), ("prefix_cache", C.c_void_p)]


class cb_step(C.Structure):
    _fields_ = [("num_reqs", C.c_int32), ("num_tokens", C.c_int32), ("num_decodes", C.c_int32),
                ("max_q_len", C.c_int32), ("max_seq_len", C.c_int32), ("n_stalled", C.c_int32),
                ("first_rejected", C.c_int32), ("held_by_margin", C.c_int32), ("prefix_sharing", C.c_int32),
                ("used_pages", C.c_int32 * CB_MAX_LAYERS), ("table_width", C.c_int32 * CB_MAX_LAYERS),
                ("off_query_start_loc", C.c_int64), ("off_seq_lens", C.c_int64), ("off_req_index", C.c_int64),
                ("off_stalled", C.c_int64), ("off_block_table", C.c_int64 * CB_MAX_LAYERS),
                ("off_slot_mapping", C.c_int64 * CB_MAX_LAYERS), ("off_ring_len", C.c_int64 * CB_MAX_LAYERS),
                ("off_matched", C.c_int64), ("used", C.c_int64)]


class cb_attn_shape(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("dtype", C.c_int32), ("window_left", C.c_int32),
                ("decode_split", C.c_int32), ("prefill_split", C.c_int32), ("prefill_rows", C.c_int32)]


class cb_plan(C.Structure):
    _fields_ = [("n_decode", C.c_int32), ("n_prefill", C.c_int32), ("n_rowwise", C.c_int32),
                ("n_combine", C.c_int32), ("n_partials", C.c_int32), ("decode_split", C.c_int32),
                ("prefill_split", C.c_int32), ("prefill_tokens", C.c_int32), ("num_tokens", C.c_int32),
                ("max_page_index", C.c_int32), ("off_decode", C.c_int64), ("off_prefill", C.c_int64),
                ("off_rowwise", C.c_int64), ("off_combine", C.c_int64), ("used", C.c_int64)]


class cb_attn_args(C.Structure):
    _fields_ = [("out", C.c_void_p), ("q", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("layout", C.c_int32), ("block_table", C.c_void_p), ("plan", C.c_void_p), ("plan_info", cb_plan),
                ("shape", cb_attn_shape), ("num_pages", C.c_int32), ("table_width", C.c_int32),
                ("scale", C.c_float), ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("phases", C.c_int32), ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("slot_mapping", C.c_void_p),
                ("num_new", C.c_int32), ("counts", C.c_void_p), ("timing_start", C.c_void_p),
                ("timing_stop", C.c_void_p)]


EXPORTS = ("cb_build_metadata", "cb_build_step", "cb_advance", "cb_slot_mapping", "cb_validate_metadata", "cb_plan_attention", "cb_kv_append", "cb_kv_copy_pages", "cb_paged_attention", "cb_paged_attention_noalloc",
           "cb_paged_attention_workspace_size", "cb_fnv1a64", "cb_block_hashes", "cb_pcache_create",
           "cb_pcache_destroy", "cb_pcache_match", "cb_pcache_lookup", "cb_pcache_allocate", "cb_pcache_commit", "cb_pcache_release",
           "cb_pcache_stats", "cb_pcache_page_info", "cb_status_str", "cb_abi_version")

_lib = None


def load(path: str = LIB_PATH):
    """Load libcb.so (built in-tree by `python -m paged_kv_attention_varlen_amd.build`). Raises if it is missing:
    there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_attention_varlen_amd.build`")
    # torch first: the library then binds to the HIP runtime torch already loaded, so device pointers and streams
    # from torch tensors are valid in the library's launches (one runtime per process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(path)
    lib.cb_build_metadata.restype = C.c_int32
    lib.cb_build_metadata.argtypes = [C.POINTER(cb_req), C.c_int32, C.POINTER(cb_sched_params),
                                      C.POINTER(cb_layer_pool), i32p, C.c_int64, C.POINTER(cb_step)]
    lib.cb_build_step.restype = C.c_int32
    lib.cb_build_step.argtypes = [C.POINTER(cb_req), C.c_int32, C.POINTER(cb_sched_params), C.POINTER(cb_layer_pool),
                                  C.POINTER(cb_attn_shape), C.c_void_p, C.c_int64, C.c_int64, C.POINTER(cb_step),
                                  C.POINTER(cb_plan), C.POINTER(C.c_int64)]
    lib.cb_advance.restype = C.c_int32
    lib.cb_advance.argtypes = [C.POINTER(cb_req), C.c_int32, C.POINTER(cb_sched_params), C.POINTER(cb_layer_pool),
                               i32p, C.POINTER(cb_step), i32p, C.c_int32]
    lib.cb_plan_attention.restype = C.c_int32
    lib.cb_plan_attention.argtypes = [i32p, i32p, i32p, C.c_int32, C.POINTER(cb_attn_shape), i32p, C.c_int64,
                                      C.POINTER(cb_plan)]
    lib.cb_kv_append.restype = C.c_int32
    lib.cb_kv_append.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                 C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]
    lib.cb_slot_mapping.restype = C.c_int32
    lib.cb_slot_mapping.argtypes = [i32p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, i32p]
    lib.cb_validate_metadata.restype = C.c_int32
    lib.cb_validate_metadata.argtypes = [i32p, i32p, C.c_int32, i32p, C.c_int32, i32p, i32p, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32, i32p, i32p]
    lib.cb_kv_copy_pages.restype = C.c_int32
    lib.cb_kv_copy_pages.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                     C.c_int64, C.c_void_p]
    lib.cb_paged_attention.restype = C.c_int32
    lib.cb_paged_attention.argtypes = [C.POINTER(cb_attn_args), C.c_void_p]
    lib.cb_paged_attention_noalloc.restype = C.c_int32
    lib.cb_paged_attention_noalloc.argtypes = [C.POINTER(cb_attn_args), C.c_void_p]
    lib.cb_paged_attention_workspace_size.restype = C.c_size_t
    lib.cb_paged_attention_workspace_size.argtypes = [C.POINTER(cb_attn_args)]
    u64p = C.POINTER(C.c_uint64)
    lib.cb_fnv1a64.restype = C.c_uint64
    lib.cb_fnv1a64.argtypes = [C.c_void_p, C.c_int64]
    lib.cb_block_hashes.restype = C.c_int32
    lib.cb_block_hashes.argtypes = [i32p, C.c_int32, C.c_int32, u64p]
    lib.cb_pcache_create.restype = C.c_int32
    lib.cb_pcache_create.argtypes = [C.c_int32, i32p, C.c_int32, C.POINTER(C.c_void_p)]
    lib.cb_pcache_destroy.restype = None
    lib.cb_pcache_destroy.argtypes = [C.c_void_p]
    lib.cb_pcache_match.restype = C.c_int32
    lib.cb_pcache_match.argtypes = [C.c_void_p, u64p, C.c_int32, i32p, i32p]
    lib.cb_pcache_lookup.restype = C.c_int32
    lib.cb_pcache_lookup.argtypes = [C.c_void_p, u64p, C.c_int32, i32p, i32p, i32p]
    lib.cb_pcache_allocate.restype = C.c_int32
    lib.cb_pcache_allocate.argtypes = [C.c_void_p, C.c_int32, i32p]
    lib.cb_pcache_commit.restype = C.c_int32
    lib.cb_pcache_commit.argtypes = [C.c_void_p, C.c_int32, C.c_uint64]
    lib.cb_pcache_release.restype = C.c_int32
    lib.cb_pcache_release.argtypes = [C.c_void_p, i32p, C.c_int32]
    lib.cb_pcache_stats.restype = C.c_int32
    lib.cb_pcache_stats.argtypes = [C.c_void_p, i32p, i32p, i32p]
    lib.cb_pcache_page_info.restype = C.c_int32
    lib.cb_pcache_page_info.argtypes = [C.c_void_p, C.c_int32, i32p, i32p, u64p]
    lib.cb_status_str.restype = C.c_char_p
    lib.cb_status_str.argtypes = [C.c_int32]
    lib.cb_abi_version.restype = C.c_int32
    lib.cb_abi_version.argtypes = []
    if lib.cb_abi_version() != ABI_VERSION:
        raise ImportError(f"libcb.so ABI version {lib.cb_abi_version()} != binding version {ABI_VERSION}")
    _lib = lib
    return lib


class CbError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = load().cb_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")
