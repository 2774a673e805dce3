"""The seeded generators: deterministic, the stated shapes and densities, a diagonal in every row."""
import numpy as np
import pytest

from workloads import CONFIGS, bf16_bits_from_f32, custom, make_inputs

EXPECTED_PAIRS = {"tiny": 28, "small": 13056, "hunyuan": 270072, "ltx": 1892352}
EXPECTED_LQ = {"tiny": 4, "small": 32, "hunyuan": 121, "wan": 148, "ltx": 384}


@pytest.mark.parametrize("name", list(CONFIGS))
def test_mask_shapes_and_densities(name):
    inp = make_inputs(name, with_qkv=False)
    w = inp["workload"]
    m = inp["mask"]
    assert m.shape == (w.H, EXPECTED_LQ[name], w.mask_pitch) and m.dtype == np.uint8
    assert not m[:, :, w.nb:].any()
    assert set(np.unique(m).tolist()) <= {0, 1}
    q = inp["q_blocks"]
    assert np.array_equal(q, np.flatnonzero(inp["placement"] == w.r))
    assert np.all(m[:, np.arange(len(q)), q] == 1)               # the diagonal block is always selected
    if name in EXPECTED_PAIRS:
        assert int(m.sum()) == EXPECTED_PAIRS[name]
    if name == "wan":
        per_head = m[:, :, :w.nb].sum(2)
        assert np.all(per_head == per_head[:, :1])                # one row count per head
        rho = per_head[:, 0] / w.nb
        assert rho.min() >= 0.05 - 1 / w.nb and rho.max() <= 0.40 + 1 / w.nb
        assert rho.max() - rho.min() > 0.15                       # heterogeneous heads


def test_tiny_density_matches_recipe():
    m = make_inputs("tiny", with_qkv=False)["mask"][0, :, :16]
    assert m.sum() / m.size == 0.4375


def test_determinism_and_qkv_layout():
    w = custom(H=2, d=64, T=3, HW=100, b=64, G=2, r=1, k_offset_sigma=3.0)
    a, b = make_inputs(w), make_inputs(w)
    for key in ("mask", "Q", "K", "V", "placement", "q_blocks"):
        assert np.array_equal(a[key], b[key])
    assert a["Q"].shape == (2, len(a["q_blocks"]) * 64, 64)
    assert a["K"].shape == (2, w.nb * 64, 64) and a["K"].dtype == np.uint16
    assert not a["K"][:, w.N:].any() and not a["V"][:, w.N:].any()
    c = make_inputs(w, seed=12)
    assert not np.array_equal(a["K"], c["K"])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38], np.float32)
    got = bf16_bits_from_f32(x)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x7F62]
