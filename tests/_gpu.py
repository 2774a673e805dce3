"""Helpers for the GPU tests: upload a drawn workload, run the three library calls, copy results back."""
from __future__ import annotations

import math

import numpy as np
import torch

import block_sparse_attention_rank_amd as bsa


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def geometry_of(w, Lq: int) -> bsa.Geometry:
    return bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=w.G, r=w.r, Lq=Lq)


def upload(inp: dict) -> dict:
    dev = dict(mask=torch.from_numpy(inp["mask"]).cuda(),
               placement=torch.from_numpy(inp["placement"]).cuda())
    if "Q" in inp:
        dev.update(Q=to_dev_bf16(inp["Q"]), K=to_dev_bf16(inp["K"]), V=to_dev_bf16(inp["V"]))
    return dev


def run_path(inp: dict, dev: dict | None = None, slot_capacity: int | None = None, attention: bool = True):
    """Run union -> pack -> attention on the device; returns the device tensors."""
    w = inp["workload"]
    g = geometry_of(w, len(inp["q_blocks"]))
    dev = dev or upload(inp)
    u = bsa.demand_union(g, dev["mask"], dev["placement"])
    out = dict(g=g, union=u, dev=dev)
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
