"""GPU parity of the placement permutation (section 4.3) through the C ABI: sparsp_permute_blocks moves
whole blocks bit-exactly as the oracle's permute_blocks does, forward and inverse, for block sizes from 16
bytes to the hidden states of the HunyuanVideo-shaped sequence (b = 128 tokens of 3072 bf16 channels)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_rank_amd as bsa
import oracle as O
from workloads import CONFIGS, placement_contiguous, placement_periodic
from workloads.configs import placement_for

pytestmark = pytest.mark.gpu


def _placement(kind, nb, b, G, seed):
    if kind == "contiguous":
        return placement_contiguous(nb, G)
    if kind == "periodic":
        return placement_periodic(nb, b, b * max(1, nb // 5 + 1), G)
    return np.random.default_rng(seed).integers(0, G, nb).astype(np.int32)


CASES = {
    # name: (outer, nb, b, C, dtype, G, placement kind)
    "tiny_16B_blocks": (1, 37, 1, 8, np.uint16, 3, "random"),
    "d64_b64_heads": (3, 50, 64, 64, np.uint16, 4, "periodic"),
    "d128_b128_heads": (2, 29, 128, 128, np.uint16, 8, "periodic"),
    "hidden_1k_channels": (1, 40, 64, 1024, np.uint16, 8, "random"),
    "ragged_chunk_tail": (1, 17, 8, 1000, np.uint16, 5, "random"),   # 16,000-byte blocks: partial 16 KiB chunk
    "fp32_rows": (2, 33, 16, 12, np.float32, 6, "contiguous"),
    "one_block": (1, 1, 64, 64, np.uint16, 1, "contiguous"),
}


def _to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda()
    return torch.from_numpy(x).cuda()


def _to_host(t, dtype):
    a = t.cpu().numpy()
    return a.view(np.uint16) if dtype == np.uint16 else a


@pytest.mark.parametrize("case", list(CASES))
def test_permute_blocks_bit_exact(require_gpu, case):
    outer, nb, b, C, dtype, G, kind = CASES[case]
    rng = np.random.default_rng(len(case))
    P = _placement(kind, nb, b, G, 7)
    pos, offs = bsa.placement_permutation(P, G)
    if dtype == np.uint16:
        x = rng.integers(0, 2**16, (outer, nb * b, C), dtype=np.uint16)
    else:
        x = rng.standard_normal((outer, nb * b, C)).astype(np.float32)
    xd, posd = _to_dev(x), torch.from_numpy(pos).cuda()
    y = bsa.permute_blocks(xd, posd, b)
    z = bsa.permute_blocks(y, posd, b, inverse=True)
    torch.cuda.synchronize()
    want = O.permute_blocks(x, pos, b)
    assert np.array_equal(_to_host(y, dtype), want)
    assert np.array_equal(_to_host(z, dtype), x)
    want_inv = O.permute_blocks(x, pos, b, inverse=True)
    w = bsa.permute_blocks(xd, posd, b, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(_to_host(w, dtype), want_inv)


def test_out_of_range_pos_moves_nothing(require_gpu):
    """A pos entry outside [0, nb) is skipped by the kernel: its destination keeps what it held."""
    nb, b, C = 6, 4, 8
    x = np.arange(nb * b * C, dtype=np.uint16).reshape(1, nb * b, C)
    pos = np.array([5, 4, -1, 2, 1, 0], np.int32)          # entry 2 is not a block index
    out = torch.full((1, nb * b, C), -1, dtype=torch.int16, device="cuda")
    bsa.permute_blocks(_to_dev(x), torch.from_numpy(pos).cuda(), b, out=out)
    torch.cuda.synchronize()
    y = out.cpu().numpy().view(np.uint16)
    for j in range(nb):
        if pos[j] >= 0:
            assert np.array_equal(y[0, pos[j] * b:(pos[j] + 1) * b], x[0, j * b:(j + 1) * b])
    assert np.all(y[0, 3 * b:4 * b] == 0xFFFF)            # block 3 has no source: untouched


def test_hidden_states_full_size(require_gpu):
    """Hidden states of the HunyuanVideo-shaped sequence under its periodic placement: [929*128][3072] bf16
    (730 MB).  Sampled blocks against the oracle's rule, every block against the inverse round trip."""
    w = CONFIGS["hunyuan"]
    C = w.H * w.d
    P = placement_for(w)
    pos, offs = bsa.placement_permutation(P, w.G)
    opos, _ = O.placement_permutation(P, w.G)
    assert np.array_equal(pos, opos)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    x = torch.randint(-2**15, 2**15, (w.nb * w.b, C), dtype=torch.int16, device="cuda", generator=g)
    posd = torch.from_numpy(pos).cuda()
    y = bsa.permute_blocks(x, posd, w.b)
    z = bsa.permute_blocks(y, posd, w.b, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(z, x)
    rng = np.random.default_rng(0)
    for j in sorted({0, w.nb - 1, *rng.integers(0, w.nb, 12).tolist()}):
        p = int(opos[j])
        assert torch.equal(y[p * w.b:(p + 1) * w.b], x[j * w.b:(j + 1) * w.b]), j
    # rank 0's shard of the permuted rows is its local query blocks in order
    qb = O.local_query_blocks(P, 0)
    shard = y[:int(offs[1]) * w.b].view(len(qb), w.b, C)
    for k in (0, len(qb) // 2, len(qb) - 1):
        j = int(qb[k])
        assert torch.equal(shard[k], x[j * w.b:(j + 1) * w.b])
