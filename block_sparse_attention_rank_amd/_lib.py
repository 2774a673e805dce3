"""ctypes loader for libsparsp.so and the C declarations of include/sparsp.h.

The library is built in-tree by ``block_sparse_attention_rank_amd.build``.  Loading fails loudly when it
is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SPARSP_LIB", os.path.join(_PKG, "libsparsp.so"))

SPARSP_OK = 0
SPARSP_ERR_INVALID = 1
SPARSP_ERR_UNSUPPORTED = 2
SPARSP_ERR_HIP = 3

# every symbol include/sparsp.h declares
EXPORTS = (
    "sparsp_abi_version",
    "sparsp_status_string",
    "sparsp_last_error",
    "sparsp_local_query_blocks",
    "sparsp_demand_union",
    "sparsp_pack_kv",
    "sparsp_block_sparse_attn",
    "sparsp_block_sparse_attn_segment",
    "sparsp_merge_partial",
    "sparsp_block_sparse_attn_segment_accumulate",
    "sparsp_chunk_plan",
    "sparsp_block_sparse_attn_chunk_accumulate",
    "sparsp_placement_permutation",
    "sparsp_permute_blocks",
    "sparsp_demand_counts",
    "sparsp_comm_volume",
    "sparsp_pool_blocks",
    "sparsp_materialize_mask",
)
# every symbol include/sparsp_measure.h declares (measurement support)
MEASURE_EXPORTS = (
    "sparsp_clock_sampler",
    "sparsp_wall_timestamp",
    "sparsp_wall_clock_khz",
)


class Geometry(ctypes.Structure):
    """sparsp_geometry: heads, head dim, block size, real tokens, ranks, this rank, local query blocks."""
    _fields_ = [("H", ctypes.c_int32), ("d", ctypes.c_int32), ("b", ctypes.c_int32), ("N", ctypes.c_int32),
                ("G", ctypes.c_int32), ("r", ctypes.c_int32), ("Lq", ctypes.c_int32)]

    @property
    def nb(self) -> int:
        return -(-self.N // self.b)

    @property
    def W(self) -> int:
        return -(-self.nb // 64)


class Chunk(ctypes.Structure):
    """sparsp_chunk: heads [h_lo, h_hi) of source rank p's segment = packed slots [slot_lo, slot_hi)."""
    _fields_ = [("p", ctypes.c_int32), ("h_lo", ctypes.c_int32), ("h_hi", ctypes.c_int32),
                ("slot_lo", ctypes.c_int32), ("slot_hi", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("tiles", ctypes.c_int64)]


class SparspError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_rank_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    gp = ctypes.POINTER(Geometry)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.sparsp_abi_version.restype = i32
    lib.sparsp_abi_version.argtypes = []
    lib.sparsp_status_string.restype = ctypes.c_char_p
    lib.sparsp_status_string.argtypes = [i32]
    lib.sparsp_last_error.restype = ctypes.c_char_p
    lib.sparsp_last_error.argtypes = []
    lib.sparsp_local_query_blocks.restype = i32
    lib.sparsp_local_query_blocks.argtypes = [i32p, i32, i32, i32, i32p, i32, i32p]
    lib.sparsp_demand_union.restype = i32
    lib.sparsp_demand_union.argtypes = [gp, P, i64, P, P, P, P, P, P, P]
    lib.sparsp_pack_kv.restype = i32
    lib.sparsp_pack_kv.argtypes = [gp, P, P, P, P, P, i32, P, P]
    lib.sparsp_block_sparse_attn.restype = i32
    lib.sparsp_block_sparse_attn.argtypes = [gp, P, P, i64, P, P, i32, f32, P, P, P]
    lib.sparsp_block_sparse_attn_segment.restype = i32
    lib.sparsp_block_sparse_attn_segment.argtypes = [gp, P, P, i64, P, P, i32, i32, f32, P, P, P]
    lib.sparsp_block_sparse_attn_segment_accumulate.restype = i32
    lib.sparsp_block_sparse_attn_segment_accumulate.argtypes = [gp, P, P, i64, P, P, i32, i32, f32, P, P, P]
    lib.sparsp_chunk_plan.restype = i32
    lib.sparsp_chunk_plan.argtypes = [i32p, i32p, i32p, i32, i32, i32, i32, i32, i32, P, i32, i32p]
    lib.sparsp_block_sparse_attn_chunk_accumulate.restype = i32
    lib.sparsp_block_sparse_attn_chunk_accumulate.argtypes = [gp, P, P, i64, P, P, i32, i32, i32, i32, f32, P, P, P]
    lib.sparsp_merge_partial.restype = i32
    lib.sparsp_merge_partial.argtypes = [gp, P, P, P, P, P]
    lib.sparsp_placement_permutation.restype = i32
    lib.sparsp_placement_permutation.argtypes = [i32p, i32, i32, i32p, i32p]
    lib.sparsp_permute_blocks.restype = i32
    lib.sparsp_permute_blocks.argtypes = [P, P, i64, i32, i64, P, i32, P]
    lib.sparsp_demand_counts.restype = i32
    lib.sparsp_demand_counts.argtypes = [gp, P, i64, P, P]
    lib.sparsp_comm_volume.restype = i32
    lib.sparsp_comm_volume.argtypes = [P, i32, i32, i32, i32p, P, P, P]
    lib.sparsp_pool_blocks.restype = i32
    lib.sparsp_pool_blocks.argtypes = [gp, P, i32, P, P, P]
    lib.sparsp_materialize_mask.restype = i32
    lib.sparsp_materialize_mask.argtypes = [gp, P, P, f32, f32, i32, P, i64, P]
    lib.sparsp_clock_sampler.restype = i32
    lib.sparsp_clock_sampler.argtypes = [P, i32, i32, P]
    lib.sparsp_wall_timestamp.restype = i32
    lib.sparsp_wall_timestamp.argtypes = [P, P]
    lib.sparsp_wall_clock_khz.restype = i32
    lib.sparsp_wall_clock_khz.argtypes = [i32p]
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SPARSP_OK:
        msg = load().sparsp_last_error().decode()
        raise SparspError(status, msg)
