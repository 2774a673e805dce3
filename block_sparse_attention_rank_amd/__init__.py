"""One sequence-parallel rank's share of block-sparse attention on MI355X (gfx950).

A thin binding over the C ABI of ``libsparsp.so`` (include/sparsp.h): torch tensors are used for device
memory and streams only, every step of the path runs in the library's HIP kernels.  The calls follow
"SparSP: Exploiting Communication Sparsity for Sequence-Parallel Video DiTs": the per-head demand union of
Eq. 2 and its compaction (sections 4.1 and 5.2), the demand-directed pack of K/V (sections 5.1, 6.1 and
6.2) and block-sparse attention with an online softmax (sections 2.2 and 2.3).
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import numpy as np

from ._lib import EXPORTS, LIB_PATH, Chunk, Geometry, SparspError, check, load  # noqa: F401

__all__ = ["Geometry", "SparspError", "UnionResult", "geometry", "local_query_blocks", "demand_union",
           "pack_kv", "block_sparse_attn", "block_sparse_attn_segment", "block_sparse_attn_segment_accumulate",
           "merge_partial", "segment_ranges", "chunk_plan", "block_sparse_attn_chunk_accumulate", "Chunk",
           "placement_permutation", "permute_blocks", "demand_counts", "comm_volume", "pool_blocks",
           "materialize_mask", "load", "LIB_PATH", "EXPORTS"]


def geometry(H: int, d: int, b: int, N: int, G: int, r: int, Lq: int) -> Geometry:
    return Geometry(H, d, b, N, G, r, Lq)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> ctypes.c_void_p:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _require(t, name, dtype, shape=None):
    """Type, dtype, shape and layout of a tensor argument.  Every call checks all of its tensors this way
    first and their device (_on_device) last, then calls the library."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _require_mask(mask, g: Geometry, name="mask"):
    """The rank's mask rows: uint8 [H][Lq][pitch] with pitch >= nb and a multiple of 16."""
    import torch
    if not isinstance(mask, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if mask.dim() != 3 or mask.shape[0] != g.H or mask.shape[1] != g.Lq:
        raise ValueError(f"{name} must be [H={g.H}][Lq={g.Lq}][pitch], got {tuple(mask.shape)}")
    pitch = mask.shape[2]
    if pitch < g.nb or pitch % 16:
        raise ValueError(f"{name} pitch must be >= nb = {g.nb} and a multiple of 16, got {pitch}")
    _require(mask, name, torch.uint8, (g.H, g.Lq, pitch))


def _require_packed(packed, g: Geometry, min_slots: int = 1, name="packed"):
    """The compacted buffer: bf16 [slots][2][b*d] with at least `min_slots` slots."""
    import torch
    if not isinstance(packed, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if packed.dim() != 3 or packed.shape[1] != 2 or packed.shape[2] != g.b * g.d:
        raise ValueError(f"{name} must be [slots][2][b*d = {g.b * g.d}], got {tuple(packed.shape)}")
    if packed.shape[0] < max(1, min_slots):
        raise ValueError(f"{name} holds {packed.shape[0]} slots, needs at least {max(1, min_slots)}")
    _require(packed, name, torch.bfloat16, tuple(packed.shape))


def _require_outputs(out, g: Geometry):
    """(O, lse): float32 [H][Lq*b][d] and [H][Lq*b]."""
    import torch
    if not isinstance(out, (tuple, list)) or len(out) != 2:
        raise TypeError("out must be a pair (O, lse)")
    O, lse = out
    _require(O, "O", torch.float32, (g.H, g.Lq * g.b, g.d))
    _require(lse, "lse", torch.float32, (g.H, g.Lq * g.b))
    return O, lse


def local_query_blocks(placement: np.ndarray, G: int, r: int) -> np.ndarray:
    """Q_r = {i : P(i) = r}, ascending (host call)."""
    P = np.ascontiguousarray(placement, dtype=np.int32)
    out = np.empty(len(P), dtype=np.int32)
    n = ctypes.c_int32(0)
    i32p = ctypes.POINTER(ctypes.c_int32)
    check(load().sparsp_local_query_blocks(P.ctypes.data_as(i32p), len(P), G, r, out.ctypes.data_as(i32p),
                                           len(out), ctypes.byref(n)))
    return out[:n.value].copy()


@dataclass
class UnionResult:
    demand: "torch.Tensor"        # int64 view of uint64 words [H][W]
    seg_offsets: "torch.Tensor"   # int32 [G*H + 1]
    slot_block: "torch.Tensor"    # int32 [H*nb]
    slot_head: "torch.Tensor"     # int32 [H*nb]
    slot_of: "torch.Tensor"       # int32 [H][nb]


def empty_union(g: Geometry, device="cuda") -> UnionResult:
    import torch
    nb, W = g.nb, g.W
    return UnionResult(
        demand=torch.empty((g.H, W), dtype=torch.int64, device=device),
        seg_offsets=torch.empty(g.G * g.H + 1, dtype=torch.int32, device=device),
        slot_block=torch.empty(g.H * nb, dtype=torch.int32, device=device),
        slot_head=torch.empty(g.H * nb, dtype=torch.int32, device=device),
        slot_of=torch.empty((g.H, nb), dtype=torch.int32, device=device),
    )


def demand_union(g: Geometry, mask, placement, out: UnionResult | None = None, stream=None) -> UnionResult:
    """Per-head demand union and per-peer compaction (sparsp_demand_union)."""
    import torch
    _require_mask(mask, g)
    _require(placement, "placement", torch.int32, (g.nb,))
    if out is None:
        out = empty_union(g, mask.device)
    else:
        _require(out.demand, "demand", torch.int64, (g.H, g.W))
        _require(out.seg_offsets, "seg_offsets", torch.int32, (g.G * g.H + 1,))
        _require(out.slot_block, "slot_block", torch.int32, (g.H * g.nb,))
        _require(out.slot_head, "slot_head", torch.int32, (g.H * g.nb,))
        _require(out.slot_of, "slot_of", torch.int32, (g.H, g.nb))
    _on_device(mask=mask, placement=placement, demand=out.demand, seg_offsets=out.seg_offsets,
               slot_block=out.slot_block, slot_head=out.slot_head, slot_of=out.slot_of)
    check(load().sparsp_demand_union(ctypes.byref(g), _ptr(mask), mask.shape[2], _ptr(placement), _ptr(out.demand),
                                     _ptr(out.seg_offsets), _ptr(out.slot_block), _ptr(out.slot_head),
                                     _ptr(out.slot_of), _stream(stream)))
    return out


def pack_kv(g: Geometry, K, V, u: UnionResult, slot_capacity: int | None = None, out=None, stream=None):
    """Gather the demanded K/V blocks into the compacted buffer (sparsp_pack_kv).

    Returns ``packed`` as a bfloat16 tensor [slot_capacity][2][b*d]; the default capacity is H*nb."""
    import torch
    shape = (g.H, g.nb * g.b, g.d)
    _require(K, "K", torch.bfloat16, shape)
    _require(V, "V", torch.bfloat16, shape)
    _require(u.seg_offsets, "seg_offsets", torch.int32, (g.G * g.H + 1,))
    _require(u.slot_block, "slot_block", torch.int32, (g.H * g.nb,))
    _require(u.slot_head, "slot_head", torch.int32, (g.H * g.nb,))
    cap = slot_capacity if slot_capacity is not None else g.H * g.nb
    if out is None:
        if cap < 1:
            raise ValueError("slot_capacity must be >= 1")
        out = torch.empty((cap, 2, g.b * g.d), dtype=torch.bfloat16, device=K.device)
    else:
        _require_packed(out, g)
        cap = out.shape[0]
    _on_device(K=K, V=V, seg_offsets=u.seg_offsets, slot_block=u.slot_block, slot_head=u.slot_head, packed=out)
    check(load().sparsp_pack_kv(ctypes.byref(g), _ptr(K), _ptr(V), _ptr(u.seg_offsets), _ptr(u.slot_block),
                                _ptr(u.slot_head), cap, _ptr(out), _stream(stream)))
    return out


def block_sparse_attn(g: Geometry, Q, mask, slot_of, packed, softmax_scale: float | None = None,
                      out=None, stream=None):
    """Block-sparse flash attention over the compacted K/V (sparsp_block_sparse_attn).

    Returns (O float32 [H][Lq*b][d], lse float32 [H][Lq*b])."""
    import torch
    _require(Q, "Q", torch.bfloat16, (g.H, g.Lq * g.b, g.d))
    _require_mask(mask, g)
    _require(slot_of, "slot_of", torch.int32, (g.H, g.nb))
    _require_packed(packed, g)
    scale = 1.0 / math.sqrt(g.d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        O = torch.empty((g.H, g.Lq * g.b, g.d), dtype=torch.float32, device=Q.device)
        lse = torch.empty((g.H, g.Lq * g.b), dtype=torch.float32, device=Q.device)
    else:
        O, lse = _require_outputs(out, g)
    _on_device(Q=Q, mask=mask, slot_of=slot_of, packed=packed, O=O, lse=lse)
    check(load().sparsp_block_sparse_attn(ctypes.byref(g), _ptr(Q), _ptr(mask), mask.shape[2], _ptr(slot_of),
                                          _ptr(packed), packed.shape[0], scale, _ptr(O), _ptr(lse),
                                          _stream(stream)))
    return O, lse


def _attn_outputs(g: Geometry, Q, out):
    import torch
    if out is None:
        return (torch.empty((g.H, g.Lq * g.b, g.d), dtype=torch.float32, device=Q.device),
                torch.empty((g.H, g.Lq * g.b), dtype=torch.float32, device=Q.device))
    return _require_outputs(out, g)


def block_sparse_attn_segment(g: Geometry, Q, mask, slot_of, packed, slot_lo: int, slot_hi: int,
                              softmax_scale: float | None = None, out=None, stream=None):
    """Attention over the selected blocks whose slot lies in [slot_lo, slot_hi)
    (sparsp_block_sparse_attn_segment).  Returns the partial (O, lse)."""
    import torch
    _require(Q, "Q", torch.bfloat16, (g.H, g.Lq * g.b, g.d))
    _require_mask(mask, g)
    _require(slot_of, "slot_of", torch.int32, (g.H, g.nb))
    _require_packed(packed, g, min_slots=slot_hi)
    scale = 1.0 / math.sqrt(g.d) if softmax_scale is None else float(softmax_scale)
    O, lse = _attn_outputs(g, Q, out)
    _on_device(Q=Q, mask=mask, slot_of=slot_of, packed=packed, O=O, lse=lse)
    check(load().sparsp_block_sparse_attn_segment(ctypes.byref(g), _ptr(Q), _ptr(mask), mask.shape[2],
                                                  _ptr(slot_of), _ptr(packed), int(slot_lo), int(slot_hi), scale,
                                                  _ptr(O), _ptr(lse), _stream(stream)))
    return O, lse


def block_sparse_attn_segment_accumulate(g: Geometry, Q, mask, slot_of, packed, slot_lo: int, slot_hi: int, O, lse,
                                         softmax_scale: float | None = None, stream=None):
    """Fold the attention over the selected blocks whose slot lies in [slot_lo, slot_hi) into the running
    (O, lse) in place (sparsp_block_sparse_attn_segment_accumulate); start from (0, -inf)."""
    import torch
    _require(Q, "Q", torch.bfloat16, (g.H, g.Lq * g.b, g.d))
    _require_mask(mask, g)
    _require(slot_of, "slot_of", torch.int32, (g.H, g.nb))
    _require_packed(packed, g, min_slots=slot_hi)
    _require_outputs((O, lse), g)
    scale = 1.0 / math.sqrt(g.d) if softmax_scale is None else float(softmax_scale)
    _on_device(Q=Q, mask=mask, slot_of=slot_of, packed=packed, O=O, lse=lse)
    check(load().sparsp_block_sparse_attn_segment_accumulate(ctypes.byref(g), _ptr(Q), _ptr(mask), mask.shape[2],
                                                             _ptr(slot_of), _ptr(packed), int(slot_lo), int(slot_hi),
                                                             scale, _ptr(O), _ptr(lse), _stream(stream)))
    return O, lse


def chunk_plan(seg_offsets: np.ndarray, counts: np.ndarray, placement: np.ndarray, G: int, r: int,
               chunks_steady: int = 1, chunks_drain: int = 1) -> list[dict]:
    """The consumption schedule of the payload (sparsp_chunk_plan, host call): a list of chunks
    {p, h_lo, h_hi, slot_lo, slot_hi, tiles} in execution order.  ``seg_offsets`` int32 [G*H+1] and
    ``counts`` int32 [H][nb] are host copies of sparsp_demand_union's and sparsp_demand_counts' outputs."""
    seg = np.ascontiguousarray(seg_offsets, dtype=np.int32)
    cnt = np.ascontiguousarray(counts, dtype=np.int32)
    P = np.ascontiguousarray(placement, dtype=np.int32)
    if cnt.ndim != 2 or cnt.shape[1] != len(P):
        raise ValueError("counts must be [H][nb] with nb = len(placement)")
    H, nb = cnt.shape
    if seg.shape != (G * H + 1,):
        raise ValueError(f"seg_offsets must hold G*H + 1 = {G * H + 1} entries")
    cap = G * H
    buf = (Chunk * cap)()
    n = ctypes.c_int32(0)
    i32p = ctypes.POINTER(ctypes.c_int32)
    check(load().sparsp_chunk_plan(seg.ctypes.data_as(i32p), cnt.ctypes.data_as(i32p), P.ctypes.data_as(i32p), G, H, nb,
                                   r, chunks_steady, chunks_drain, buf, cap, ctypes.byref(n)))
    return [dict(p=c.p, h_lo=c.h_lo, h_hi=c.h_hi, slot_lo=c.slot_lo, slot_hi=c.slot_hi, tiles=c.tiles)
            for c in buf[:n.value]]


def block_sparse_attn_chunk_accumulate(g: Geometry, Q, mask, slot_of, packed, chunk: dict, O, lse,
                                       softmax_scale: float | None = None, stream=None):
    """Fold one chunk of a schedule (heads [h_lo, h_hi), slots [slot_lo, slot_hi)) into the running (O, lse) in
    place (sparsp_block_sparse_attn_chunk_accumulate); only that head range is launched."""
    import torch
    _require(Q, "Q", torch.bfloat16, (g.H, g.Lq * g.b, g.d))
    _require_mask(mask, g)
    _require(slot_of, "slot_of", torch.int32, (g.H, g.nb))
    _require_packed(packed, g, min_slots=chunk["slot_hi"])
    _require_outputs((O, lse), g)
    scale = 1.0 / math.sqrt(g.d) if softmax_scale is None else float(softmax_scale)
    _on_device(Q=Q, mask=mask, slot_of=slot_of, packed=packed, O=O, lse=lse)
    check(load().sparsp_block_sparse_attn_chunk_accumulate(ctypes.byref(g), _ptr(Q), _ptr(mask), mask.shape[2],
                                                           _ptr(slot_of), _ptr(packed), int(chunk["slot_lo"]),
                                                           int(chunk["slot_hi"]), int(chunk["h_lo"]), int(chunk["h_hi"]),
                                                           scale, _ptr(O), _ptr(lse), _stream(stream)))
    return O, lse


def merge_partial(g: Geometry, O, lse, O_part, lse_part, stream=None):
    """Fold the partial result (O_part, lse_part) into (O, lse) in place (sparsp_merge_partial)."""
    import torch
    for t, name in ((O, "O"), (O_part, "O_part")):
        _require(t, name, torch.float32, (g.H, g.Lq * g.b, g.d))
    for t, name in ((lse, "lse"), (lse_part, "lse_part")):
        _require(t, name, torch.float32, (g.H, g.Lq * g.b))
    _on_device(O=O, lse=lse, O_part=O_part, lse_part=lse_part)
    check(load().sparsp_merge_partial(ctypes.byref(g), _ptr(O), _ptr(lse), _ptr(O_part), _ptr(lse_part),
                                      _stream(stream)))
    return O, lse


def segment_ranges(seg_offsets: np.ndarray, H: int, G: int) -> list[tuple[int, int]]:
    """Slot range [lo, hi) of every source rank's segment, from the host copy of seg_offsets (each
    source rank's heads are consecutive)."""
    s = np.asarray(seg_offsets)
    return [(int(s[p * H]), int(s[(p + 1) * H])) for p in range(G)]


def placement_permutation(placement: np.ndarray, G: int) -> tuple[np.ndarray, np.ndarray]:
    """Rank-major block order (sparsp_placement_permutation, host call): returns pos int32 [nb] (the
    permuted position of logical block j) and rank_offsets int32 [G+1]."""
    P = np.ascontiguousarray(placement, dtype=np.int32)
    pos = np.empty(len(P), dtype=np.int32)
    offs = np.empty(G + 1, dtype=np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    check(load().sparsp_placement_permutation(P.ctypes.data_as(i32p), len(P), G, pos.ctypes.data_as(i32p),
                                              offs.ctypes.data_as(i32p)))
    return pos, offs


def permute_blocks(x, pos, b: int, inverse: bool = False, out=None, stream=None):
    """Move whole blocks of b rows of x [..., nb*b, C] (sparsp_permute_blocks): out[..., pos[j]] = x[..., j]
    or, with ``inverse``, out[..., j] = x[..., pos[j]].  ``pos`` is a device int32 tensor [nb]."""
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous device tensor of at least 2 dimensions")
    rows, C = x.shape[-2], x.shape[-1]
    if rows % b:
        raise ValueError("the row count must be a multiple of b")
    nb = rows // b
    _require(pos, "pos", torch.int32, (nb,))
    outer = x.numel() // max(1, rows * C)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must match x")
    _on_device(pos=pos, out=out)
    check(load().sparsp_permute_blocks(_ptr(x), _ptr(out), outer, nb, b * C * x.element_size(), _ptr(pos),
                                       1 if inverse else 0, _stream(stream)))
    return out


def demand_counts(g: Geometry, mask, out=None, stream=None):
    """Access counts of the rank's mask rows (sparsp_demand_counts): int32 [H][nb], the number of local
    query blocks selecting each key block."""
    import torch
    _require_mask(mask, g)
    if out is None:
        out = torch.empty((g.H, g.nb), dtype=torch.int32, device=mask.device)
    else:
        _require(out, "counts", torch.int32, (g.H, g.nb))
    _on_device(mask=mask, counts=out)
    check(load().sparsp_demand_counts(ctypes.byref(g), _ptr(mask), mask.shape[2], _ptr(out), _stream(stream)))
    return out


def comm_volume(demand_all: np.ndarray, placement: np.ndarray, G: int) -> dict:
    """Block counts of demand-directed delivery, the relaying ring and the dense ring (sparsp_comm_volume,
    host call).  demand_all: uint64 (or int64) [G][H][W], consumer c's demand words."""
    D = np.ascontiguousarray(demand_all).view(np.uint64)
    if D.ndim != 3 or D.shape[0] != G:
        raise ValueError("demand_all must be [G][H][W]")
    P = np.ascontiguousarray(placement, dtype=np.int32)
    H, W = D.shape[1], D.shape[2]
    if W != -(-len(P) // 64):
        raise ValueError("demand words do not match the placement length")
    direct = np.empty((G, G), np.int64)
    relay = np.empty((G, G), np.int64)
    dense = np.empty(G, np.int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    check(load().sparsp_comm_volume(D.ctypes.data, G, H, len(P), P.ctypes.data_as(i32p), direct.ctypes.data,
                                    relay.ctypes.data, dense.ctypes.data))
    return dict(direct=direct, relay=relay, dense=dense)


def pool_blocks(g: Geometry, X, block_ids=None, out=None, stream=None):
    """Block means of the real rows (sparsp_pool_blocks): X bf16 [H][n*b][d] -> float32 [H][n][d].
    ``block_ids`` (device int32 [n]) names each block's logical id; None means block k is block k."""
    import torch
    _require(X, "X", torch.bfloat16)
    if X.dim() != 3 or X.shape[0] != g.H or X.shape[2] != g.d or X.shape[1] % g.b:
        raise ValueError("X must be [H][n*b][d]")
    n = X.shape[1] // g.b
    if block_ids is not None:
        _require(block_ids, "block_ids", torch.int32, (n,))
    if out is None:
        out = torch.empty((g.H, n, g.d), dtype=torch.float32, device=X.device)
    else:
        _require(out, "pooled", torch.float32, (g.H, n, g.d))
    _on_device(X=X, block_ids=block_ids, pooled=out)
    check(load().sparsp_pool_blocks(ctypes.byref(g), _ptr(X), n, _ptr(block_ids), _ptr(out), _stream(stream)))
    return out


def materialize_mask(g: Geometry, q_pooled, k_pooled, tau: float, k_min: int, softmax_scale: float | None = None,
                     out=None, stream=None):
    """Block mask [H][Lq][64*W] uint8 of the rank's rows from pooled tiles (sparsp_materialize_mask):
    Top-p at CDF threshold ``tau`` with a Top-k floor ``k_min``."""
    import torch
    _require(q_pooled, "q_pooled", torch.float32, (g.H, g.Lq, g.d))
    _require(k_pooled, "k_pooled", torch.float32, (g.H, g.nb, g.d))
    scale = 1.0 / math.sqrt(g.d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((g.H, g.Lq, 64 * g.W), dtype=torch.uint8, device=q_pooled.device)
    else:
        _require_mask(out, g)
    _on_device(q_pooled=q_pooled, k_pooled=k_pooled, mask=out)
    check(load().sparsp_materialize_mask(ctypes.byref(g), _ptr(q_pooled), _ptr(k_pooled), scale, float(tau),
                                         int(k_min), _ptr(out), out.shape[2], _stream(stream)))
    return out
