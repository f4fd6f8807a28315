"""ctypes loader of libcsa2.so: struct layouts and prototypes of include/csa2.h."""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "csa2.h")

c_int32, c_void_p, c_float, c_size_t = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

CSA2_OK, CSA2_ERR_INVALID_ARG, CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP = 0, 1, 2, 3, 4
CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2
KCLASS_APPEND, KCLASS_SCAN, KCLASS_SELECT, KCLASS_ATTN, KCLASS_DENSE = 0, 1, 2, 3, 4
KCLASS_POOL_SCAN, KCLASS_POOL_SELECT = 5, 6
NUM_KCLASSES = 7
DTYPE_F32, DTYPE_BF16 = 0, 1
MAX_K, MAX_H_IDX, MAX_H, MIN_PAGE_SIZE = 2048, 16, 128, 64
STATIC_SCRATCH_BYTES = 64 << 20
STEP_DENSE_INDEX, STEP_POOL, STEP_ATTN_PER_HEAD_GROUP, STEP_PRUNE = 1, 2, 4, 8
PRUNE_BLOCK, PRUNE_BOUND_BYTES = 64, 256
DENSE_RESCORE_ALL = -1


class CacheView(ctypes.Structure):
    _fields_ = [("kv", c_void_p), ("idx_k", c_void_p), ("page_table", c_void_p), ("seq_lens", c_void_p),
                ("num_pages", c_int32), ("page_size", c_int32), ("num_seqs", c_int32), ("max_pages", c_int32),
                ("idxk_bounds", c_void_p)]


class TimingRing(ctypes.Structure):
    _fields_ = [("start", ctypes.POINTER(c_void_p)), ("stop", ctypes.POINTER(c_void_p)),
                ("capacity", c_int32), ("count", c_int32)]


class Timing(ctypes.Structure):
    _fields_ = [("ring", ctypes.POINTER(TimingRing) * NUM_KCLASSES)]


class StepArgs(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(CacheView)),
                ("new_slots", c_void_p), ("new_kv", c_void_p), ("new_idxk", c_void_p), ("n_new", c_int32),
                ("q_idx", c_void_p), ("w", c_void_p), ("h_idx", c_int32),
                ("q", c_void_p), ("h", c_int32), ("sm_scale", c_float),
                ("q_seq", c_void_p), ("q_vis", c_void_p), ("nq", c_int32), ("k", c_int32), ("max_vis", c_int32),
                ("idx", c_void_p), ("cnt", c_void_p), ("out", c_void_p), ("lse", c_void_p),
                ("ws", c_void_p), ("ws_bytes", c_size_t), ("flags", ctypes.c_uint32),
                ("pool", c_void_p), ("pool_cnt", c_void_p), ("pool_k", c_int32),
                ("dense_cand_factor", c_int32), ("timing", ctypes.POINTER(Timing)),
                ("seed", c_void_p), ("seed_cnt", c_void_p)]


GROUP_MAX_LAYERS, GROUP_MAX_AUX = 64, 4


class GroupExec(ctypes.Structure):
    _fields_ = [("aux", c_void_p * GROUP_MAX_AUX), ("n_aux", c_int32),
                ("events", ctypes.POINTER(c_void_p)), ("n_events", c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp4_kv_cache_layer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.csa2_append_quant_fp4.argtypes = [P(CacheView), c_void_p, c_void_p, c_void_p, c_int32, c_void_p]
    lib.csa2_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]
    lib.csa2_workspace_bytes.restype = c_size_t
    lib.csa2_workspace_init.argtypes = [c_void_p, c_size_t, c_void_p]
    lib.csa2_index_topk.argtypes = [P(CacheView), c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                    c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.csa2_prefill_index_topk.argtypes = lib.csa2_index_topk.argtypes
    lib.csa2_pool_index_topk.argtypes = [P(CacheView), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                         c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.csa2_pool_workspace_bytes.argtypes = [c_int32, c_int32]
    lib.csa2_pool_workspace_bytes.restype = c_size_t
    lib.csa2_sparse_attn.argtypes = [P(CacheView), c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                     c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.csa2_layer_step.argtypes = [c_int32, P(StepArgs), c_void_p]
    lib.csa2_layer_step_static.argtypes = [c_int32, P(StepArgs), c_void_p]
    lib.csa2_lse_merge.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                   c_void_p]
    lib.csa2_fake_quant_fp4.argtypes = [c_void_p, c_void_p, ctypes.c_int64, c_int32, c_void_p]
    lib.csa2_group_events.argtypes = [c_int32, c_int32]
    lib.csa2_group_events.restype = c_int32
    lib.csa2_group_step.argtypes = [c_int32, P(c_int32), P(StepArgs), c_void_p, P(GroupExec)]
    lib.csa2_idxk_bounds_build.argtypes = [P(CacheView), c_int32, c_int32, c_void_p]
    lib.csa2_status_string.argtypes = [c_int32]
    lib.csa2_status_string.restype = ctypes.c_char_p
    for fn in ("csa2_append_quant_fp4", "csa2_workspace_init", "csa2_index_topk", "csa2_prefill_index_topk",
               "csa2_pool_index_topk", "csa2_sparse_attn",
               "csa2_layer_step", "csa2_layer_step_static", "csa2_group_step", "csa2_lse_merge", "csa2_fake_quant_fp4",
               "csa2_idxk_bounds_build"):
        getattr(lib, fn).restype = c_int32
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions include/csa2.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", txt)))


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().csa2_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != CSA2_OK:
        raise Csa2Error(fn, status)
