"""Pins for the oracle's block-sparse attention (CPU only).

The oracle is compared with an independent library routine (torch's scaled_dot_product_attention in
float64 on the CPU, given an explicit boolean token mask), with special cases that reduce to textbook
results (all-ones mask = dense attention; identity block mask = per-block local attention; uniform and
one-hot softmax), and with invariants (weights sum to one, O is reconstructed from lse, padding and
placement do not change the result).  A few tests plant a mistake in a copy of the oracle and check that
the pins catch it.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from workloads import custom, make_inputs


def _f64(x):
    return torch.from_numpy(O.bf16_to_f64(x))


def _sdpa_reference(inp, h, k):
    """torch SDPA (float64, CPU) for local query block k of head h, with the token mask built here by
    comparing each query/key token pair's block ids against the mask row."""
    w = inp["workload"]
    b, N = w.b, w.N
    q = _f64(inp["Q"][h, k * b:(k + 1) * b])
    K = _f64(inp["K"][h, :N])
    V = _f64(inp["V"][h, :N])
    key_block = np.arange(N) // b
    allowed = inp["mask"][h, k][key_block] != 0                  # [N]
    attn = torch.from_numpy(np.broadcast_to(allowed, (b, N)).copy())
    if not allowed.any():
        return None
    out = torch.nn.functional.scaled_dot_product_attention(
        q[None, None], K[None, None], V[None, None], attn_mask=attn[None, None], scale=1.0 / math.sqrt(w.d))
    return out[0, 0].numpy()


def _check_against_sdpa(inp, attention_fn=O.attention_block, atol=1e-12):
    w = inp["workload"]
    scale = 1.0 / math.sqrt(w.d)
    worst = 0.0
    for h in range(w.H):
        for k in range(len(inp["q_blocks"])):
            ref = _sdpa_reference(inp, h, k)
            got, _ = attention_fn(inp["Q"], inp["K"], inp["V"], inp["mask"], h, k, w.b, w.N, scale)
            if ref is None:
                continue
            worst = max(worst, float(np.abs(got - ref).max()))
    return worst <= atol, worst


@pytest.mark.parametrize("kind", ["ones", "topk", "box"])
def test_matches_library_sdpa(kind):
    """Section 2.2: softmax(QK^T/sqrt(d))V, restricted to the allowed key tokens."""
    w = custom(H=2, d=64, T=3, HW=128, b=64, G=3, r=1, mask_kind=kind, density=0.4)
    ok, worst = _check_against_sdpa(make_inputs(w))
    assert ok, worst


def test_all_ones_equals_dense_attention():
    """With every block selected the method is plain dense attention over the real tokens."""
    w = custom(H=1, d=64, T=2, HW=160, b=64, G=2, r=0, mask_kind="ones")
    inp = make_inputs(w)
    Oo, lse = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, 1 / math.sqrt(w.d))
    q = _f64(inp["Q"][0])
    K = _f64(inp["K"][0, :w.N])
    V = _f64(inp["V"][0, :w.N])
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None], V[None], scale=1 / math.sqrt(w.d))
    rows = O.real_rows(inp["q_blocks"], w.b, w.N)
    assert np.abs(Oo[0][rows] - ref[0].numpy()[rows]).max() < 1e-12
    ref_lse = torch.logsumexp((q @ K.T) / math.sqrt(w.d), dim=1).numpy()
    assert np.abs(lse[0][rows] - ref_lse[rows]).max() < 1e-12


def test_identity_mask_is_local_block_attention():
    """An identity block mask makes every query block attend to its own block only: independent b x b
    dense attention per block."""
    w = custom(H=2, d=64, T=2, HW=256, b=64, G=4, r=2, mask_kind="identity")
    inp = make_inputs(w)
    Oo, _ = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, 1 / math.sqrt(w.d))
    for h in range(w.H):
        for k, i in enumerate(inp["q_blocks"]):
            q = _f64(inp["Q"][h, k * w.b:(k + 1) * w.b])
            kk = _f64(inp["K"][h, i * w.b:(i + 1) * w.b])
            vv = _f64(inp["V"][h, i * w.b:(i + 1) * w.b])
            ref = torch.nn.functional.scaled_dot_product_attention(q[None], kk[None], vv[None],
                                                                   scale=1 / math.sqrt(w.d))[0].numpy()
            assert np.abs(Oo[h, k * w.b:(k + 1) * w.b] - ref).max() < 1e-12


def test_weights_sum_to_one_and_lse_reconstructs_output():
    w = custom(H=2, d=64, T=3, HW=192, b=64, G=3, r=0, density=0.3)
    inp = make_inputs(w)
    scale = 1 / math.sqrt(w.d)
    Oo, lse = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, scale)
    for h in range(w.H):
        for k in range(len(inp["q_blocks"])):
            toks = O.allowed_keys(inp["mask"][h, k], w.nb, w.b, w.N)
            q = O.bf16_to_f64(inp["Q"][h, k * w.b:(k + 1) * w.b])
            s = q @ O.bf16_to_f64(inp["K"][h, toks]).T * scale
            p = np.exp(s - lse[h, k * w.b:(k + 1) * w.b, None])
            assert np.abs(p.sum(1) - 1).max() < 1e-12
            recon = p @ O.bf16_to_f64(inp["V"][h, toks])
            assert np.abs(recon - Oo[h, k * w.b:(k + 1) * w.b]).max() < 1e-12


def test_identical_keys_give_the_mean_of_values():
    """Equal logits give uniform weights, so O is the mean of the allowed V rows."""
    w = custom(H=1, d=64, T=2, HW=128, b=64, G=2, r=0, density=0.5)
    inp = make_inputs(w)
    inp["K"][:] = inp["K"][0, 0]                     # every key row identical
    Oo, _ = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, 1 / math.sqrt(w.d))
    for k in range(len(inp["q_blocks"])):
        toks = O.allowed_keys(inp["mask"][0, k], w.nb, w.b, w.N)
        mean = O.bf16_to_f64(inp["V"][0, toks]).mean(0)
        assert np.abs(Oo[0, k * w.b:(k + 1) * w.b] - mean[None]).max() < 1e-12


def test_one_dominant_key_selects_its_value():
    """A key whose logit exceeds all others by a wide margin takes all the weight (to 1e-12)."""
    from workloads import bf16_bits_from_f32
    w = custom(H=1, d=64, T=2, HW=128, b=64, G=2, r=0, mask_kind="ones")
    inp = make_inputs(w)
    q = np.zeros((w.b, w.d), np.float32)
    q[:, 0] = 1.0
    inp["Q"][0, :w.b] = bf16_bits_from_f32(q)
    K = np.zeros((w.nb * w.b, w.d), np.float32)
    K[77, 0] = 50 * math.sqrt(w.d)                   # logit 50 for key 77, 0 for the rest
    inp["K"][0] = bf16_bits_from_f32(K)
    Oo, lse = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, 1 / math.sqrt(w.d))
    v77 = O.bf16_to_f64(inp["V"][0, 77])
    assert np.abs(Oo[0, :w.b] - v77[None]).max() < 1e-12 * 1e9 * math.exp(-50) + 1e-12
    assert np.abs(lse[0, :w.b] - 50.0).max() < 1e-12


def test_empty_row_gives_zero_and_minus_inf():
    w = custom(H=1, d=64, T=2, HW=128, b=64, G=2, r=0, mask_kind="zeros")
    inp = make_inputs(w)
    Oo, lse = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, 0.125)
    assert np.all(Oo == 0) and np.all(np.isneginf(lse))


def test_padding_matches_unpadded_sequence():
    """N not a multiple of b: the zero tail of the last block must not take part.  The same tokens
    with a larger T (so the tail becomes real zero tokens) would differ; the N-token library result
    must match."""
    w = custom(H=2, d=64, T=3, HW=100, b=64, G=2, r=1, mask_kind="ones")   # N = 300, nb = 5, pad 20
    assert w.N % w.b
    ok, worst = _check_against_sdpa(make_inputs(w))
    assert ok, worst


def test_placement_does_not_change_results():
    """Section 4.3: the placement permutes whole blocks and leaves block membership alone, so a logical
    query block gets the same output under either placement (same logical mask, same values)."""
    base = dict(H=2, d=64, T=4, HW=256, b=64, G=4, mask_kind="topk", density=0.3)
    res = {}
    for placement in ("contiguous", "periodic"):
        for r in range(4):
            w = custom(placement=placement, r=r, **base)
            inp = make_inputs(w)
            Oo, _ = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, 1 / math.sqrt(w.d))
            for k, i in enumerate(inp["q_blocks"]):
                res.setdefault(int(i), []).append((inp["mask"][:, k, :w.nb].copy(), Oo[:, k * 64:(k + 1) * 64]))
    for i, outs in res.items():
        assert len(outs) == 2
        (m0, o0), (m1, o1) = outs
        assert np.array_equal(m0, m1)          # the generator's mask is a function of logical blocks
        assert np.abs(o0 - o1).max() < 1e-13


def test_dense_token_mask_self_check():
    """The blockwise oracle equals the dense formula with a kron(M, ones(b, b)) token mask."""
    w = make_inputs("tiny")["workload"]
    inp = make_inputs("tiny")
    scale = 1 / math.sqrt(w.d)
    Oo, lse = O.attention(inp["Q"], inp["K"], inp["V"], inp["mask"], w.b, w.N, scale)
    for h in range(w.H):
        tm = O.token_mask(inp["mask"][h], inp["q_blocks"], w.b, w.N)
        Od, lsed, wts = O.dense_masked_attention(O.bf16_to_f64(inp["Q"][h]), O.bf16_to_f64(inp["K"][h]),
                                                 O.bf16_to_f64(inp["V"][h]), tm, scale)
        assert np.abs(Od - Oo[h]).max() < 1e-12
        assert np.abs(lsed - lse[h]).max() < 1e-12
        assert np.abs(wts.sum(1) - 1).max() < 1e-12


# ------------------------------------------------------------------------------ planted mistakes


def _planted_no_scale(Q, K, V, mask, h, k, b, N, scale):
    return O.attention_block(Q, K, V, mask, h, k, b, N, 1.0)


def _planted_keeps_padding(Q, K, V, mask, h, k, b, N, scale):
    nb = -(-N // b)
    return O.attention_block(Q, K, V, mask, h, k, b, nb * b, scale)


def _planted_transposed_mask(Q, K, V, mask, h, k, b, N, scale):
    m = mask.copy()
    m[h, :, :m.shape[1]] = m[h, :, :m.shape[1]].T if m.shape[1] <= m.shape[2] else m[h]
    return O.attention_block(Q, K, V, m, h, k, b, N, scale)


@pytest.mark.parametrize("planted", [_planted_no_scale, _planted_keeps_padding, _planted_transposed_mask])
def test_pins_catch_planted_mistakes(planted):
    w = custom(H=1, d=64, T=3, HW=100, b=64, G=1, r=0, mask_kind="topk", density=0.5)
    inp = make_inputs(w)
    assert _check_against_sdpa(inp)[0]
    assert not _check_against_sdpa(inp, attention_fn=planted)[0]
