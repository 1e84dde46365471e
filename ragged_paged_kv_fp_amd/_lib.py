"""ctypes view of libfp.so (the C ABI in include/fp.h). No torch here."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp.so")

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_u64 = ctypes.c_uint64
c_ptr = ctypes.c_void_p

FP_OK = 0
FP_ERR_NULL = -1
FP_ERR_SHAPE = -2
FP_ERR_UNSUPPORTED = -3
FP_ERR_WORKSPACE = -4
FP_ERR_HIP = -5
ERR_NAMES = {FP_ERR_NULL: "FP_ERR_NULL", FP_ERR_SHAPE: "FP_ERR_SHAPE", FP_ERR_UNSUPPORTED: "FP_ERR_UNSUPPORTED",
             FP_ERR_WORKSPACE: "FP_ERR_WORKSPACE", FP_ERR_HIP: "FP_ERR_HIP"}

FP_ST_SLOT_RANGE = 1
FP_ST_FROZEN = 2
FP_ST_KVLEN = 4
FP_ST_FOLD_CLAMP = 8
FP_ST_READOUT_RANGE = 16
FP_ST_MASK_SHORT = 32
FP_ST_PAGE_RANGE = 64
FP_ST_PLAN_MISMATCH = 128
FP_ST_ADAPTER = 256
FP_ST_DUP_WRITE = 512
FP_ST_SHARED_CELL = 1024

FP_FOLD_ALL = -1
FP_FOLD_CHANNEL = -2

EXPORTS = ("fp_append_kv", "fp_attend_workspace_bytes", "fp_attend", "fp_attend_noalloc",
           "fp_attend_noalloc_max_bytes", "fp_hazard_workspace_bytes",
           "fp_check_hazards", "fp_fold", "fp_readout", "fp_fold_readout", "fp_attn_mass",
           "fp_advance", "fp_tova_mask", "fp_lora_workspace_bytes", "fp_adapter_lora", "fp_adapter_ia3",
           "fp_vertical_merge", "fp_kv_bytes", "fp_pages_for", "fp_page_waste", "fp_page_bytes", "fp_version",
           "fp_source_hash")


class FpGeometry(ctypes.Structure):
    _fields_ = [("num_lanes", c_i32), ("num_rows", c_i32), ("indptr", c_ptr), ("indptr_host", c_ptr),
                ("positions", c_ptr), ("slots", c_ptr), ("kv_len", c_ptr), ("fold", c_ptr)]


class FpKvPool(ctypes.Structure):
    _fields_ = [("kv", c_ptr), ("num_pages", c_i32), ("page_size", c_i32), ("num_kv_heads", c_i32),
                ("head_dim", c_i32), ("page_indptr", c_ptr), ("page_indptr_host", c_ptr), ("page_ids", c_ptr),
                ("committed_len", c_ptr)]


class FpMask(ctypes.Structure):
    _fields_ = [("bits", c_ptr), ("word_offset", c_ptr), ("word_offset_host", c_ptr)]


class FpLora(ctypes.Structure):
    _fields_ = [("num_adapters", ctypes.c_int32), ("rank", ctypes.c_int32), ("d_in", ctypes.c_int32),
                ("d_out", ctypes.c_int32), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class FpTuning(ctypes.Structure):
    _fields_ = [("decode_split_slots", c_i32), ("reserved", c_i32 * 7), ("attn_begin", c_ptr), ("attn_end", c_ptr),
                ("prefill_end", c_ptr), ("merge_end", c_ptr)]


class FpError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code} ({ERR_NAMES.get(code, 'unknown')})")
        self.code = code


_lib = None


class StaleLibraryError(ImportError):
    """libfp.so was compiled from other sources than the ones in the tree."""


def check_fresh(lib: ctypes.CDLL, sources=None) -> None:
    """Raise StaleLibraryError unless the library's compiled-in source hash equals
    the hash of the current sources (so no test or benchmark runs an old binary)."""
    from . import build

    lib.fp_source_hash.argtypes = []
    lib.fp_source_hash.restype = ctypes.c_char_p
    built = lib.fp_source_hash().decode()
    now = build.source_hash(sources)
    if built != now:
        raise StaleLibraryError(f"libfp.so was built from other sources (built {built[:12]}, tree {now[:12]}): "
                                "rebuild it with `python -m ragged_paged_kv_fp_amd.build` or __graft_entry__.build()")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp.so; raises if it has not been built or is older than its
    sources (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m ragged_paged_kv_fp_amd.build` "
                          "(or __graft_entry__.build()); the step has no CPU fallback")
    lib = ctypes.CDLL(path)
    check_fresh(lib)
    P = ctypes.POINTER
    lib.fp_append_kv.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, c_ptr, ctypes.c_float, c_ptr, c_ptr]
    lib.fp_append_kv.restype = c_i32
    lib.fp_attend_workspace_bytes.argtypes = [P(FpKvPool), P(FpGeometry), P(FpMask), c_i32, P(FpTuning)]
    lib.fp_attend_workspace_bytes.restype = c_i64
    lib.fp_attend.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, c_i32, ctypes.c_float, ctypes.c_float, P(FpMask),
                              c_ptr, c_ptr, c_ptr, ctypes.c_size_t, P(FpTuning), c_ptr, c_ptr]
    lib.fp_attend.restype = c_i32
    lib.fp_attend_noalloc.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, c_i32, ctypes.c_float, ctypes.c_float,
                                      P(FpMask), c_ptr, c_ptr, P(FpTuning), c_ptr, c_ptr]
    lib.fp_attend_noalloc.restype = c_i32
    lib.fp_attend_noalloc_max_bytes.argtypes = []
    lib.fp_attend_noalloc_max_bytes.restype = c_i64
    lib.fp_hazard_workspace_bytes.argtypes = [P(FpKvPool)]
    lib.fp_hazard_workspace_bytes.restype = c_i64
    lib.fp_check_hazards.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, ctypes.c_size_t, c_ptr, c_ptr]
    lib.fp_check_hazards.restype = c_i32
    lib.fp_fold.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, c_ptr, c_ptr]
    lib.fp_fold.restype = c_i32
    lib.fp_readout.argtypes = [P(FpGeometry), c_ptr, c_i32, c_ptr, c_i32, c_ptr, c_ptr, c_ptr]
    lib.fp_readout.restype = c_i32
    lib.fp_fold_readout.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, c_ptr, c_i32, c_ptr, c_i32, c_ptr, c_ptr,
                                    c_ptr]
    lib.fp_fold_readout.restype = c_i32
    lib.fp_attn_mass.argtypes = [P(FpKvPool), P(FpGeometry), c_i32, P(FpMask), c_ptr, c_ptr, ctypes.c_size_t, P(FpTuning),
                                 c_ptr, c_ptr]
    lib.fp_attn_mass.restype = c_i32
    lib.fp_lora_workspace_bytes.argtypes = [P(FpGeometry), P(FpLora)]
    lib.fp_lora_workspace_bytes.restype = ctypes.c_int64
    lib.fp_adapter_lora.argtypes = [P(FpGeometry), P(FpLora), c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, ctypes.c_size_t,
                                    c_ptr, c_ptr]
    lib.fp_adapter_lora.restype = c_i32
    lib.fp_adapter_ia3.argtypes = [P(FpGeometry), c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr]
    lib.fp_adapter_ia3.restype = c_i32
    lib.fp_advance.argtypes = [P(FpKvPool), P(FpGeometry), c_ptr, c_ptr, c_ptr, c_ptr, c_ptr]
    lib.fp_advance.restype = c_i32
    lib.fp_tova_mask.argtypes = [P(FpKvPool), P(FpGeometry)] + [c_ptr] * 10 + [c_ptr]  # ..., status, stream
    lib.fp_tova_mask.restype = c_i32
    lib.fp_vertical_merge.argtypes = [c_i32] + [c_ptr] * 10 + [c_i32] + [c_ptr] * 6  # L, 10 inputs, page_size, 6 outputs
    lib.fp_vertical_merge.restype = c_i32
    lib.fp_kv_bytes.argtypes = [c_i32, c_i32, c_i32, c_u64, c_i32]
    lib.fp_kv_bytes.restype = c_u64
    lib.fp_pages_for.argtypes = [c_u64, c_i32]
    lib.fp_pages_for.restype = c_u64
    lib.fp_page_waste.argtypes = [c_u64, c_i32]
    lib.fp_page_waste.restype = c_u64
    lib.fp_page_bytes.argtypes = [c_i32, c_i32, c_i32]
    lib.fp_page_bytes.restype = c_u64
    lib.fp_version.argtypes = []
    lib.fp_version.restype = ctypes.c_char_p
    _lib = lib
    return lib
