"""Helpers for the GPU tests: upload a drawn workload, run the library calls, copy results back, and compare
attention outputs with the oracle over many (head, query block) items on the host's cores."""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import block_sparse_attention_rank_amd as bsa
import oracle as O


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def geometry_of(w, Lq: int) -> bsa.Geometry:
    return bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=w.G, r=w.r, Lq=Lq)


def local_blocks(inp: dict) -> np.ndarray:
    """Q_r through the C ABI (sparsp_local_query_blocks); must equal the generator's ascending {i : P(i) = r}."""
    w = inp["workload"]
    q = bsa.local_query_blocks(inp["placement"], w.G, w.r)
    assert np.array_equal(q, inp["q_blocks"]), "sparsp_local_query_blocks disagrees with {i : P(i) = r}"
    return q


def upload(inp: dict) -> dict:
    dev = dict(mask=torch.from_numpy(inp["mask"]).cuda(),
               placement=torch.from_numpy(inp["placement"]).cuda())
    if "Q" in inp:
        dev.update(Q=to_dev_bf16(inp["Q"]), K=to_dev_bf16(inp["K"]), V=to_dev_bf16(inp["V"]))
    return dev


def run_path(inp: dict, dev: dict | None = None, slot_capacity: int | None = None, attention: bool = True):
    """Run the local set (host), union -> pack -> attention (device); returns the device tensors."""
    w = inp["workload"]
    q_blocks = local_blocks(inp)
    g = geometry_of(w, len(q_blocks))
    dev = dev or upload(inp)
    u = bsa.demand_union(g, dev["mask"], dev["placement"])
    out = dict(g=g, union=u, dev=dev, q_blocks=q_blocks)
    if "K" in dev:
        out["packed"] = bsa.pack_kv(g, dev["K"], dev["V"], u, slot_capacity=slot_capacity)
        if attention:
            out["O"], out["lse"] = bsa.block_sparse_attn(g, dev["Q"], dev["mask"], u.slot_of, out["packed"],
                                                         1.0 / math.sqrt(w.d))
    torch.cuda.synchronize()
    return out


def union_host(u) -> dict:
    S = int(u.seg_offsets[-1].item())
    return dict(demand=u.demand.cpu().numpy().view(np.uint64), seg_offsets=u.seg_offsets.cpu().numpy(),
                slot_block=u.slot_block[:S].cpu().numpy(), slot_head=u.slot_head[:S].cpu().numpy(),
                slot_of=u.slot_of.cpu().numpy(), S=S)


def oracle_workers() -> int:
    """Threads for the oracle comparisons: the host's cores, at most 16 (the GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare_items(inp: dict, O_dev: np.ndarray, lse_dev: np.ndarray, items, segment: int | None = None) -> dict:
    """Compare the device (O, lse) with the oracle on every listed (head, query block), in parallel threads
    (NumPy releases the GIL inside its kernels; BLAS runs one thread per call).  With ``segment`` = p the
    oracle is restricted to the keys of the blocks rank p owns.  Returns the absolute O errors over real rows
    (max, sum, count), the largest relative lse error and the number of rows whose finiteness differs or
    whose O is nonzero where the oracle's row is empty."""
    from threadpoolctl import threadpool_limits

    w = inp["workload"]
    b, scale = w.b, 1.0 / math.sqrt(w.d)

    def one(item):
        h, k = item
        if segment is None:
            Oo, lo = O.attention_block(inp["Q"], inp["K"], inp["V"], inp["mask"], h, k, b, w.N, scale)
        else:
            Oo, lo = O.attention_block_segment(inp["Q"], inp["K"], inp["V"], inp["mask"], inp["placement"], segment,
                                               h, k, b, w.N, scale)
        rows = O.real_rows(inp["q_blocks"][k:k + 1], b, w.N)
        got = O_dev[h, k * b:(k + 1) * b][rows]
        e = np.abs(got - Oo[rows])
        gl, ol = lse_dev[h, k * b:(k + 1) * b][rows], lo[rows]
        fin = np.isfinite(ol)
        bad = int(np.count_nonzero(np.isfinite(gl) != fin)) + int(np.count_nonzero(got[~fin]))
        le = float(np.max(np.abs(gl[fin] - ol[fin]) / np.maximum(1.0, np.abs(ol[fin])))) if fin.any() else 0.0
        return float(e.max()) if e.size else 0.0, float(e.sum()), int(e.size), le, bad

    with threadpool_limits(1), ThreadPoolExecutor(oracle_workers()) as ex:
        res = list(ex.map(one, items))
    mx = max((r[0] for r in res), default=0.0)
    n = sum(r[2] for r in res)
    return dict(max=mx, mean=sum(r[1] for r in res) / max(1, n), count=n, items=len(res),
                lse_rel=max((r[3] for r in res), default=0.0), bad_rows=sum(r[4] for r in res))


def all_items(inp: dict):
    w = inp["workload"]
    return [(h, k) for h in range(w.H) for k in range(len(inp["q_blocks"]))]
