"""Five video-DiT-shaped workloads for one rank's share of block-sparse attention, plus small custom ones.

Geometry.  A video latent of T frames x HW tokens per frame is flattened in raster order (frame, row,
column) into N = T*HW tokens, cut into blocks of b tokens (nb = ceil(N/b); the last block is zero-padded).
The SparSP paper (full text, section 4.3, Eq. 4) places blocks on G sequence-parallel ranks; rank r owns
the query blocks Q_r = {i : P(i) = r}.  Two placements are drawn here:

* contiguous: P(j) = floor(j*G/nb), the default partition the paper calls naive (sections 3.2 and 8.3);
* periodic (Eq. 4): P(j) = floor(G*s/B) for a block at in-frame position s of B positions per frame.
  For frames whose token count is not a multiple of b, a block is located by its centre token
  c = j*b + b/2, so P(j) = floor(G*(c mod HW)/HW) in integer arithmetic; for frame-aligned blocks and
  G dividing B this equals Eq. 4 exactly.

Masks.  Only the rank's own rows M[h, i in Q_r, :] are drawn (uint8 0/1, rows padded with zeros to a
pitch of 64-column words).  Section 4.3 of the paper reports diagonal (intra-frame), multi-diagonal
(same region across frames) and column patterns; the synthetic masks model the first two with a
distance D(i, j) = |s_i - s_j| + b*|t_i - t_j| between block centres (t = frame, s = in-frame token
offset) and add per-head random blocks:

* box:  every j with |t_i - t_j| <= 1 and |s_i - s_j| <= b, plus ``n_random`` random blocks outside it;
* topk: K_row blocks per row: the K_row - ceil(K_row/8) nearest by (D, j), then ceil(K_row/8) random
  blocks among the rest.  The diagonal block (D = 0) is always present, so real rows are never empty.

Values.  Q, K, V are N(0, 1) float32 draws rounded to bfloat16 (round to nearest even), returned as
uint16 bit patterns.  K may carry a per-(head, block) mean offset mu ~ N(0, sigma^2) added before
rounding.  Rows at token index >= N are zero.

Seeds.  Every stream is a ``numpy.random.SeedSequence([seed, stream, ...])``: stream 0 = Q (per head and
logical block, so a block's Q does not depend on placement), 1 = K, 2 = V (per head), 3 = mask random
picks (per head and logical query block), 4 = per-head densities, 5 = K block offsets.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_MASK, STREAM_DENSITY, STREAM_KOFF = range(6)


@dataclass(frozen=True)
class Workload:
    name: str
    H: int            # heads
    d: int            # head dim
    T: int            # frames
    HW: int           # tokens per frame
    b: int            # tokens per block
    G: int            # sequence-parallel ranks (virtual on one GPU)
    r: int = 0        # the rank whose share is computed
    placement: str = "contiguous"           # "contiguous" | "periodic"
    mask_kind: str = "topk"                 # "box" | "topk" | "ones" | "identity" | "zeros"
    density: float = 0.2                    # topk: K_row = max(k_floor, round(density*nb))
    density_range: tuple | None = None      # topk: per-head density ~ U(lo, hi)
    k_floor: int = 0
    n_random: int = 2                       # box: random blocks outside the window
    k_offset_sigma: float = 0.0             # std of per-(head, block) mean offsets added to K
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.T * self.HW

    @property
    def nb(self) -> int:
        return -(-self.N // self.b)

    @property
    def W(self) -> int:
        return -(-self.nb // 64)

    @property
    def mask_pitch(self) -> int:
        return 64 * self.W


CONFIGS: dict[str, Workload] = {
    "tiny": Workload("tiny", H=1, d=64, T=4, HW=16 * 16, b=64, G=4, placement="contiguous",
                     mask_kind="box", n_random=2, seed=1,
                     note="1 head, d 64, 4x16x16 tokens, block 64, 4 ranks; +-1 block box + 2 random"),
    "small": Workload("small", H=8, d=64, T=16, HW=32 * 32, b=64, G=8, placement="contiguous",
                      mask_kind="topk", density=0.20, seed=2,
                      note="8 heads, d 64, 16x32x32 tokens, block 64, 8 ranks; window + random, 20%"),
    "hunyuan": Workload("hunyuan", H=24, d=128, T=33, HW=45 * 80, b=128, G=8, placement="periodic",
                        mask_kind="topk", density=0.10, seed=3,
                        note="HunyuanVideo-shaped: 24 heads, d 128, 33x45x80 tokens, block 128, 8 ranks, "
                             "periodic placement; window + per-head random, 10%"),
    "wan": Workload("wan", H=40, d=128, T=21, HW=45 * 80, b=128, G=4, placement="contiguous",
                    mask_kind="topk", density_range=(0.05, 0.40), seed=4,
                    note="Wan-14B-shaped: 40 heads, d 128, 21x45x80 tokens, block 128, 4 ranks; "
                         "per-head density U(5%, 40%)"),
    "ltx": Workload("ltx", H=32, d=64, T=32, HW=64 * 96, b=64, G=8, placement="contiguous",
                    mask_kind="topk", density=0.05, k_floor=16, k_offset_sigma=3.0, seed=5,
                    note="LTX-Video-shaped: 32 heads, d 64, 32x64x96 tokens, block 64, 8 ranks; 5% with a "
                         "top-k floor of 16; K block mean offsets N(0, 9)"),
}


def custom(name="custom", **kw) -> Workload:
    """A small workload for tests; keyword arguments override the Workload fields."""
    base = dict(H=2, d=64, T=2, HW=200, b=64, G=2, seed=11)
    base.update(kw)
    return Workload(name, **base)


# --------------------------------------------------------------------------------------------------
# placement


def placement_contiguous(nb: int, G: int) -> np.ndarray:
    j = np.arange(nb, dtype=np.int64)
    return ((j * G) // nb).astype(np.int32)


def placement_periodic(nb: int, b: int, HW: int, G: int) -> np.ndarray:
    j = np.arange(nb, dtype=np.int64)
    centre = j * b + b // 2
    return ((G * (centre % HW)) // HW).astype(np.int32)


def placement_for(w: Workload) -> np.ndarray:
    if w.placement == "contiguous":
        return placement_contiguous(w.nb, w.G)
    if w.placement == "periodic":
        return placement_periodic(w.nb, w.b, w.HW, w.G)
    raise ValueError(f"unknown placement {w.placement!r}")


# --------------------------------------------------------------------------------------------------
# masks


def _centres(w: Workload):
    c = np.arange(w.nb, dtype=np.int64) * w.b + w.b // 2
    return c // w.HW, c % w.HW          # frame, in-frame token offset


def _row_counts(w: Workload) -> np.ndarray:
    """K_row per head for the topk recipe."""
    if w.density_range is not None:
        rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_DENSITY]))
        lo, hi = w.density_range
        rho = rng.uniform(lo, hi, size=w.H)
    else:
        rho = np.full(w.H, w.density)
    k = np.maximum(w.k_floor, np.rint(rho * w.nb).astype(np.int64))
    return np.clip(k, 1, w.nb)


def _row_keys(w: Workload, h: int, qb: np.ndarray) -> np.ndarray:
    """Uniform sort keys for the random picks, one stream per (head, logical query block), so that a
    logical row's mask does not depend on which rank holds it."""
    keys = np.empty((len(qb), w.nb))
    for k, i in enumerate(qb.tolist()):
        keys[k] = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_MASK, h, i])).random(w.nb)
    return keys


def make_mask(w: Workload, q_blocks: np.ndarray) -> np.ndarray:
    H, nb, Lq = w.H, w.nb, len(q_blocks)
    mask = np.zeros((H, Lq, w.mask_pitch), dtype=np.uint8)
    if Lq == 0:
        return mask
    qb = np.asarray(q_blocks, dtype=np.int64)
    if w.mask_kind == "zeros":
        return mask
    if w.mask_kind == "ones":
        mask[:, :, :nb] = 1
        return mask
    if w.mask_kind == "identity":
        for h in range(H):
            mask[h, np.arange(Lq), qb] = 1
        return mask

    t, s = _centres(w)
    dist = np.abs(s[qb][:, None] - s[None, :]) + w.b * np.abs(t[qb][:, None] - t[None, :])  # [Lq, nb]
    if w.mask_kind == "box":
        window = (np.abs(t[qb][:, None] - t[None, :]) <= 1) & (np.abs(s[qb][:, None] - s[None, :]) <= w.b)
        for h in range(H):
            keys = _row_keys(w, h, qb)
            keys[window] = np.inf
            order = np.argsort(keys, axis=1, kind="stable")
            sel = window.copy()
            for k in range(Lq):
                avail = int((~window[k]).sum())
                sel[k, order[k, :min(w.n_random, avail)]] = True
            mask[h, :, :nb] = sel
        return mask
    if w.mask_kind != "topk":
        raise ValueError(f"unknown mask kind {w.mask_kind!r}")

    # nearest blocks by (D, j): a stable argsort of D keeps ascending j among ties
    near_order = np.argsort(dist, axis=1, kind="stable")
    k_rows = _row_counts(w)
    for h in range(H):
        K_row = int(k_rows[h])
        k_rnd = min(-(-K_row // 8), nb - 1) if nb > 1 else 0
        k_near = K_row - k_rnd
        sel = np.zeros((Lq, nb), dtype=bool)
        np.put_along_axis(sel, near_order[:, :k_near], True, axis=1)
        keys = _row_keys(w, h, qb)
        keys[sel] = np.inf
        pick = np.argsort(keys, axis=1, kind="stable")[:, :k_rnd]
        np.put_along_axis(sel, pick, True, axis=1)
        mask[h, :, :nb] = sel
    return mask


# --------------------------------------------------------------------------------------------------
# values


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _kv_head(w: Workload, stream: int, h: int, out: np.ndarray, offsets: np.ndarray | None):
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, stream, h]))
    x = rng.standard_normal((w.nb * w.b, w.d), dtype=np.float32)
    if offsets is not None:
        x += np.repeat(offsets[h].astype(np.float32), w.b)[:, None]
    x[w.N:] = 0.0
    out[h] = bf16_bits_from_f32(x)


def _q_head(w: Workload, q_blocks: np.ndarray, h: int, out: np.ndarray):
    b = w.b
    for k, i in enumerate(q_blocks):
        rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_Q, h, int(i)]))
        x = rng.standard_normal((b, w.d), dtype=np.float32)
        valid = w.N - int(i) * b
        if valid < b:
            x[max(valid, 0):] = 0.0
        out[h, k * b:(k + 1) * b] = bf16_bits_from_f32(x)


def make_qkv(w: Workload, q_blocks: np.ndarray):
    H, d, b, nb = w.H, w.d, w.b, w.nb
    Q = np.empty((H, len(q_blocks) * b, d), dtype=np.uint16)
    K = np.empty((H, nb * b, d), dtype=np.uint16)
    V = np.empty((H, nb * b, d), dtype=np.uint16)
    offsets = None
    if w.k_offset_sigma:
        rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_KOFF]))
        offsets = rng.normal(0.0, w.k_offset_sigma, size=(H, nb))
    with ThreadPoolExecutor(_workers()) as ex:
        futs = [ex.submit(_q_head, w, q_blocks, h, Q) for h in range(H)]
        futs += [ex.submit(_kv_head, w, STREAM_K, h, K, offsets) for h in range(H)]
        futs += [ex.submit(_kv_head, w, STREAM_V, h, V, None) for h in range(H)]
        for f in futs:
            f.result()
    return Q, K, V


def make_inputs(w: Workload | str, with_qkv: bool = True, **overrides) -> dict:
    """Draw one workload.  Returns host arrays:

    placement int32 [nb]; q_blocks int32 [Lq] (ascending {i : P(i) = r}); mask uint8 [H][Lq][pitch];
    and, with ``with_qkv``, Q uint16 [H][Lq*b][d], K and V uint16 [H][nb*b][d] (bfloat16 bits).
    """
    if isinstance(w, str):
        w = CONFIGS[w]
    if overrides:
        w = replace(w, **overrides)
    if not (0 <= w.r < w.G):
        raise ValueError("rank out of range")
    placement = placement_for(w)
    q_blocks = np.flatnonzero(placement == w.r).astype(np.int32)
    out = dict(workload=w, placement=placement, q_blocks=q_blocks, mask=make_mask(w, q_blocks))
    if with_qkv:
        out["Q"], out["K"], out["V"] = make_qkv(w, q_blocks)
    return out


def softmax_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
