"""GPU parity of the communication-volume accounting through the C ABI: the access-count kernel is
bit-exact against the oracle on every workload's rank share and on edge masks, and the volumes computed
from the GPU's demand unions of every consumer rank (sparsp_demand_union once per rank, then
sparsp_comm_volume) equal the oracle's, for contiguous and periodic placements and G = 2, 4, 8."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_attention_rank_amd as bsa
import oracle as O
from workloads import CONFIGS, custom, make_inputs
from workloads.configs import make_mask, placement_for

pytestmark = pytest.mark.gpu


def _geom(w, Lq, r=None):
    return bsa.geometry(H=w.H, d=w.d, b=w.b, N=w.N, G=w.G, r=w.r if r is None else r, Lq=Lq)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_counts_bit_exact(require_gpu, name):
    inp = make_inputs(name, with_qkv=False)
    w = inp["workload"]
    g = _geom(w, len(inp["q_blocks"]))
    got = bsa.demand_counts(g, torch.from_numpy(inp["mask"]).cuda()).cpu().numpy()
    assert np.array_equal(got, O.access_counts(inp["mask"], w.nb))


@pytest.mark.parametrize("kind", ["ones", "identity", "zeros", "bytes"])
def test_counts_edge_masks(require_gpu, kind):
    w = custom(H=3, T=3, HW=700, b=64, G=2, mask_kind="ones" if kind == "bytes" else kind)
    inp = make_inputs(w, with_qkv=False)
    mask = inp["mask"].copy()
    if kind == "bytes":                         # any nonzero byte selects; pitch columns are ignored
        rng = np.random.default_rng(0)
        mask[:, :, :w.nb] *= rng.integers(0, 256, mask[:, :, :w.nb].shape).astype(np.uint8)
        mask[:, :, w.nb:] = 255
    g = _geom(w, len(inp["q_blocks"]))
    got = bsa.demand_counts(g, torch.from_numpy(mask).cuda()).cpu().numpy()
    assert np.array_equal(got, O.access_counts(mask, w.nb))


def _gpu_volume(w, mask_all, P):
    words = []
    dev_all = torch.from_numpy(mask_all).cuda()
    for c in range(w.G):
        q = O.local_query_blocks(P, c)
        g = _geom(w, len(q), r=c)
        rows = dev_all[:, torch.from_numpy(q.astype(np.int64)).cuda(), :].contiguous()
        u = bsa.demand_union(g, rows, torch.from_numpy(P).cuda())
        words.append(u.demand.cpu().numpy().view(np.uint64))
    return bsa.comm_volume(np.stack(words), P, w.G), np.stack(words)


@pytest.mark.parametrize("name,G,placement", [("small", 8, "contiguous"), ("hunyuan", 2, "periodic"),
                                              ("hunyuan", 4, "contiguous"), ("hunyuan", 8, "periodic"),
                                              ("hunyuan", 8, "contiguous"), ("wan", 4, "contiguous")])
def test_volume_from_gpu_unions(require_gpu, name, G, placement):
    w = dataclasses.replace(CONFIGS[name], G=G, placement=placement)
    P = placement_for(w)
    mask_all = make_mask(w, np.arange(w.nb, dtype=np.int32))
    got, words = _gpu_volume(w, mask_all, P)
    U = np.zeros((G, w.H, w.nb), dtype=bool)
    for c in range(G):
        U[c] = O.demand_union(mask_all[:, O.local_query_blocks(P, c), :], w.nb)
        assert np.array_equal(words[c], O.demand_words(U[c]))
    want = O.comm_volume(U, P, G)
    for key in ("direct", "relay", "dense"):
        assert np.array_equal(got[key], want[key]), key
