"""Plain CPU oracle for one sequence-parallel rank's share of block-sparse attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
or call this module.  The product path (the HIP library and its Python binding) never does: it shares
no code, header, table or helper with this file, and this file imports nothing from it.

Source: "SparSP: Exploiting Communication Sparsity for Sequence-Parallel Video DiTs" (the paper's full
text as published on paperpeel.com).  What it computes, step by step:

1. The rank's local query blocks Q_r = {i : P(i) = r} (section 4.1, Eq. 2 uses Q_r; section 4.3 fixes P
   once per geometry).
2. The per-head demand union U[h] = {j : exists i in Q_r with M[h, i, j] = 1} (Eq. 2, taken over all
   owners p at once; section 5.2 "head-preserving demand": never unioned across heads).
3. The per-peer compaction: for p = 0..G-1, then h = 0..H-1, then ascending j with j in U[h] and
   P(j) = p, the next packed slot (section 5.2 "metadata-free exchange": one (head, block) enumeration
   in row-major order that both ends derive, each head a contiguous range; section 6.1: one slot region
   per peer).  Segment offsets are exclusive prefix sums of the (p, h) counts.
4. The pack: slot s holds K[h_s] rows of block j_s (b x d, token-major) followed by V[h_s] rows of block
   j_s stored transposed (d x b, key-contiguous), both bfloat16 bit patterns.  The pages say the
   selected blocks are packed contiguously and then laid out for the attention kernel on arrival
   (section 6.2); the transposed V is that layout, written at pack time.
5. Block-sparse attention: for each head and local query block, softmax(Q K^T / sqrt(d)) V over exactly
   the key tokens of the blocks the mask row selects (section 2.2 gives the dense formula; Eq. 2's block
   mask M restricts it).  Key tokens at index >= N (the zero padding of the last block) are excluded.
   An empty key set gives O = 0 and lse = -inf.  lse = m + ln(sum exp(s - m)) is the natural-log
   log-sum-exp that an online-softmax merge across pieces of KV needs (section 2.3).

Everything is fp64 on the exact values of the bfloat16 inputs.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------------------------------
# data format


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: a bfloat16 is the high half of an IEEE float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------------------
# step 1: the local set


def local_query_blocks(placement: np.ndarray, r: int) -> np.ndarray:
    """Q_r as an ascending int32 array: every logical block i with P(i) = r (section 4.1, Eq. 2)."""
    return np.array([i for i, p in enumerate(np.asarray(placement).tolist()) if p == r], dtype=np.int32)


# --------------------------------------------------------------------------------------------------
# step 2: demand union (Eq. 2, per head)


def demand_union_sets(mask: np.ndarray, nb: int) -> list[set]:
    """Brute force: U[h] as a Python set, built entry by entry (small inputs only)."""
    H, Lq = mask.shape[0], mask.shape[1]
    out = []
    for h in range(H):
        u = set()
        for k in range(Lq):
            for j in range(nb):
                if mask[h, k, j]:
                    u.add(j)
        out.append(u)
    return out


def demand_union(mask: np.ndarray, nb: int) -> np.ndarray:
    """U[h][j] = OR over the rank's rows k of M[h, k, j]; bool [H][nb]."""
    m = np.asarray(mask)[:, :, :nb] != 0
    if m.shape[1] == 0:
        return np.zeros((m.shape[0], nb), dtype=bool)
    return np.any(m, axis=1)


def demand_words(U: np.ndarray) -> np.ndarray:
    """Bit-pack U into uint64 words: bit (j mod 64) of word floor(j/64); bits past nb are 0."""
    H, nb = U.shape
    W = -(-nb // 64)
    words = np.zeros((H, W), dtype=np.uint64)
    for h in range(H):
        for j in np.flatnonzero(U[h]):
            words[h, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return words


# --------------------------------------------------------------------------------------------------
# step 3: per-peer compaction (section 5.2)


def compact(U: np.ndarray, placement: np.ndarray, G: int) -> dict:
    """Enumerate (p, h, j) in row-major order and number the demanded blocks.

    Returns seg_offsets int32 [G*H+1] (index p*H + h; the last entry is S), slot_block and slot_head
    int32 [S], slot_of int32 [H][nb] (-1 where not demanded) and S.
    """
    H, nb = U.shape
    P = np.asarray(placement)
    counts = np.zeros(G * H, dtype=np.int64)
    blocks, heads = [], []
    for p in range(G):
        owned = P == p
        for h in range(H):
            js = np.flatnonzero(U[h] & owned)          # ascending
            counts[p * H + h] = len(js)
            blocks.append(js)
            heads.append(np.full(len(js), h))
    seg = np.zeros(G * H + 1, dtype=np.int64)
    seg[1:] = np.cumsum(counts)
    slot_block = np.concatenate(blocks).astype(np.int32) if blocks else np.zeros(0, np.int32)
    slot_head = np.concatenate(heads).astype(np.int32) if heads else np.zeros(0, np.int32)
    slot_of = np.full((H, nb), -1, dtype=np.int32)
    slot_of[slot_head, slot_block] = np.arange(len(slot_block), dtype=np.int32)
    return dict(seg_offsets=seg.astype(np.int32), slot_block=slot_block, slot_head=slot_head,
                slot_of=slot_of, S=int(seg[-1]))


def compact_bruteforce(U_sets: list[set], placement, G: int, nb: int) -> dict:
    """The same enumeration with Python loops and a running counter (small inputs only)."""
    H = len(U_sets)
    seg, slot_block, slot_head = [], [], []
    slot_of = [[-1] * nb for _ in range(H)]
    s = 0
    for p in range(G):
        for h in range(H):
            seg.append(s)
            for j in range(nb):
                if j in U_sets[h] and int(placement[j]) == p:
                    slot_block.append(j)
                    slot_head.append(h)
                    slot_of[h][j] = s
                    s += 1
    seg.append(s)
    return dict(seg_offsets=np.array(seg, np.int32), slot_block=np.array(slot_block, np.int32),
                slot_head=np.array(slot_head, np.int32), slot_of=np.array(slot_of, np.int32), S=s)


def segment_range(seg_offsets: np.ndarray, H: int, p: int) -> tuple[int, int]:
    """Slots [lo, hi) of source rank p: its heads are consecutive (section 6.2, derived byte ranges)."""
    return int(seg_offsets[p * H]), int(seg_offsets[(p + 1) * H])


# --------------------------------------------------------------------------------------------------
# step 4: pack


def pack(K: np.ndarray, V: np.ndarray, slot_block: np.ndarray, slot_head: np.ndarray, b: int) -> np.ndarray:
    """packed[s, 0] = K[h_s, j_s*b:(j_s+1)*b, :] (b x d); packed[s, 1] = that V block transposed (d x b).

    Bit patterns in, bit patterns out (uint16 [S][2][b*d]).
    """
    S = len(slot_block)
    d = K.shape[2]
    out = np.empty((S, 2, b * d), dtype=np.uint16)
    for s in range(S):
        h, j = int(slot_head[s]), int(slot_block[s])
        out[s, 0] = K[h, j * b:(j + 1) * b, :].reshape(-1)
        out[s, 1] = V[h, j * b:(j + 1) * b, :].T.reshape(-1)
    return out


# --------------------------------------------------------------------------------------------------
# step 5: block-sparse attention


def _attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Exact softmax attention of query rows q over key rows k (fp64).  Returns (O, lse, weights)."""
    if k.shape[0] == 0:
        return (np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf),
                np.zeros((q.shape[0], 0)))
    s = (q @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    w = e / l
    return w @ v, (m + np.log(l))[:, 0], w


def allowed_keys(mask_row: np.ndarray, nb: int, b: int, N: int) -> np.ndarray:
    """Token indices a query block may attend to: the real tokens of every selected key block."""
    js = np.flatnonzero(np.asarray(mask_row)[:nb])
    if len(js) == 0:
        return np.zeros(0, dtype=np.int64)
    toks = (js[:, None] * b + np.arange(b)[None, :]).reshape(-1)
    return toks[toks < N]


def attention_block(Q, K, V, mask, h: int, k: int, b: int, N: int, scale: float):
    """O (b x d) and lse (b) for local query block k of head h."""
    nb = -(-N // b)
    toks = allowed_keys(mask[h, k], nb, b, N)
    q = bf16_to_f64(Q[h, k * b:(k + 1) * b])
    kk = bf16_to_f64(K[h, toks])
    vv = bf16_to_f64(V[h, toks])
    O, lse, _ = _attend(q, kk, vv, scale)
    return O, lse


def attention(Q, K, V, mask, b: int, N: int, scale: float, items=None):
    """Block-sparse attention for the rank's local queries.

    Q uint16 [H][Lq*b][d]; K, V uint16 [H][nb*b][d]; mask uint8 [H][Lq][>= nb].
    Returns O float64 [H][Lq*b][d] and lse float64 [H][Lq*b].  With ``items`` (a list of (h, k)) only
    those query blocks are computed; the others stay NaN.
    """
    H, Lq = mask.shape[0], mask.shape[1]
    d = Q.shape[2]
    O = np.full((H, Lq * b, d), np.nan)
    lse = np.full((H, Lq * b), np.nan)
    todo = items if items is not None else [(h, k) for h in range(H) for k in range(Lq)]
    for h, k in todo:
        O[h, k * b:(k + 1) * b], lse[h, k * b:(k + 1) * b] = attention_block(Q, K, V, mask, h, k, b, N, scale)
    return O, lse


def token_mask(mask_rows: np.ndarray, q_blocks: np.ndarray, b: int, N: int) -> np.ndarray:
    """Expand one head's block mask rows [Lq][nb] to a token mask [Lq*b][nb*b]: M kron ones(b, b),
    with key tokens >= N switched off."""
    nb = -(-N // b)
    m = np.kron(np.asarray(mask_rows)[:, :nb] != 0, np.ones((b, b), dtype=bool))
    m[:, N:] = False
    return m


def dense_masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, tmask: np.ndarray, scale: float):
    """The dense formula of section 2.2 with disallowed logits set to -inf (self-check only).

    q [n][d], k and v [m][d] float64; tmask bool [n][m].  Returns (O, lse, weights)."""
    s = (q @ k.T) * scale
    s = np.where(tmask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    l = e.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        w = np.where(l > 0, e / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l[:, 0] > 0, m_safe[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)), -np.inf)
    return w @ v, lse, w


# --------------------------------------------------------------------------------------------------
# comparison helpers (used by the tests and the benchmark's CPU leg)


def real_rows(q_blocks: np.ndarray, b: int, N: int) -> np.ndarray:
    """Boolean [Lq*b]: which local query rows are real tokens (< N)."""
    tok = (np.asarray(q_blocks, dtype=np.int64)[:, None] * b + np.arange(b)[None, :]).reshape(-1)
    return tok < N


# --------------------------------------------------------------------------------------------------
# segment-wise consumption (section 2.3 online softmax across pieces of KV; section 5.1 the payload of
# each source rank arrives as its own piece)


def attention_block_segment(Q, K, V, mask, placement, p: int, h: int, k: int, b: int, N: int, scale: float):
    """O and lse of local query block k of head h over the keys of the selected blocks owned by rank p
    only: the definition of attention restricted to that key set.  An empty set gives (0, -inf)."""
    nb = -(-N // b)
    row = np.array(mask[h, k, :nb], copy=True)
    row[np.asarray(placement)[:nb] != p] = 0
    toks = allowed_keys(row, nb, b, N)
    q = bf16_to_f64(Q[h, k * b:(k + 1) * b])
    O, lse, _ = _attend(q, bf16_to_f64(K[h, toks]), bf16_to_f64(V[h, toks]), scale)
    return O, lse


def lse_merge(O_a, lse_a, O_b, lse_b):
    """Combine two partial results over disjoint key sets: the log-sum-exp of the union is
    ln(e^lse_a + e^lse_b) and each part's weighted mean is weighted by its share e^(lse_part - lse).
    Rows where both parts are empty stay (0, -inf)."""
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isfinite(lse), np.exp(lse_a - lse), 0.0)
        wb = np.where(np.isfinite(lse), np.exp(lse_b - lse), 0.0)
    return wa[..., None] * O_a + wb[..., None] * O_b, lse


# --------------------------------------------------------------------------------------------------
# the consumption schedule (section 7: the local block stays whole, remote blocks are cut into chunks, finer
# for the final remote block where the pipeline drains (7.1, Figure 11); attention is partitioned by heads and
# the chunk with the highest sparsity is scheduled last (7.2))


def segment_tiles(mask: np.ndarray, placement: np.ndarray, G: int, nb: int) -> np.ndarray:
    """tiles[p][h] = number of selected (local row k, key block j) pairs of head h with j owned by rank p: the
    attention work (and the payload use) of head h's part of source rank p's segment.  Counted one by one."""
    H, Lq = mask.shape[0], mask.shape[1]
    P = [int(x) for x in np.asarray(placement).tolist()]
    tiles = np.zeros((G, H), dtype=np.int64)
    for h in range(H):
        for k in range(Lq):
            for j in np.flatnonzero(np.asarray(mask[h, k, :nb])):
                tiles[P[int(j)], h] += 1
    return tiles


def chunk_plan(seg_offsets: np.ndarray, tiles: np.ndarray, G: int, H: int, r: int, chunks_steady: int,
               chunks_drain: int) -> list[dict]:
    """The order in which rank r consumes its payload, as a list of chunks {p, h_lo, h_hi, slot_lo, slot_hi,
    tiles}.  Segments arrive in ring order p = r, r+1, ..., r+G-1 (mod G).  The local segment (p = r) is one
    chunk.  Each remote segment is cut by heads into chunks_steady chunks, the last one to arrive into
    chunks_drain chunks; c chunks over H heads (c at most H) are the head ranges [i*H//c, (i+1)*H//c).  A chunk
    holds the slots of its heads in segment p (each head of a segment is contiguous).  Within a segment the
    chunks run from the most selected tiles to the fewest (equal counts: lower heads first), so that the chunk
    with the highest sparsity is the last.  Chunks without slots carry no payload and no work and are left
    out."""
    seg = [int(x) for x in np.asarray(seg_offsets).tolist()]
    plan = []
    for k in range(G):
        p = (r + k) % G
        if k == 0:
            c = 1
        elif k == G - 1:
            c = chunks_drain
        else:
            c = chunks_steady
        c = min(c, H)
        chunks = []
        for i in range(c):
            h_lo, h_hi = i * H // c, (i + 1) * H // c
            lo, hi = seg[p * H + h_lo], seg[p * H + h_hi]
            if hi > lo:
                chunks.append(dict(p=p, h_lo=h_lo, h_hi=h_hi, slot_lo=lo, slot_hi=hi,
                                   tiles=int(sum(int(tiles[p, h]) for h in range(h_lo, h_hi)))))
        chunks.sort(key=lambda ch: (-ch["tiles"], ch["h_lo"]))
        plan.extend(chunks)
    return plan


def attention_block_slots(Q, K, V, mask, slot_of, slot_lo: int, slot_hi: int, h: int, k: int, b: int, N: int,
                          scale: float):
    """O and lse of local query block k of head h over the keys of the selected blocks whose packed slot lies
    in [slot_lo, slot_hi): the definition of attention restricted to that key set ((0, -inf) if empty)."""
    nb = -(-N // b)
    row = np.array(mask[h, k, :nb], copy=True)
    s = np.asarray(slot_of)[h, :nb]
    row[(s < slot_lo) | (s >= slot_hi)] = 0
    toks = allowed_keys(row, nb, b, N)
    q = bf16_to_f64(Q[h, k * b:(k + 1) * b])
    O, lse, _ = _attend(q, bf16_to_f64(K[h, toks]), bf16_to_f64(V[h, toks]), scale)
    return O, lse


# --------------------------------------------------------------------------------------------------
# placement permutation (section 4.3: the placement is realised as a fixed permutation of logical blocks
# to (rank, offset) pairs, applied to the hidden states before the distributed region and undone after it)


def placement_permutation(placement: np.ndarray, G: int) -> tuple[np.ndarray, np.ndarray]:
    """Rank-major order of the logical blocks: rank 0's blocks first, then rank 1's, ...; inside a rank,
    ascending logical index (the order of Q_p).  Returns pos int32 [nb] (the permuted position of logical
    block j) and rank_offsets int32 [G+1] (rank p's blocks occupy [rank_offsets[p], rank_offsets[p+1])).
    Written as the enumeration itself: a running counter over (p, j)."""
    P = [int(x) for x in np.asarray(placement).tolist()]
    nb = len(P)
    pos = [-1] * nb
    offsets = []
    n = 0
    for p in range(G):
        offsets.append(n)
        for j in range(nb):
            if P[j] == p:
                pos[j] = n
                n += 1
    offsets.append(n)
    return np.array(pos, np.int32), np.array(offsets, np.int32)


def permute_blocks(x: np.ndarray, pos: np.ndarray, b: int, inverse: bool = False) -> np.ndarray:
    """Move whole blocks of b rows: x [outer][nb*b][C] -> y with y[o, pos[j]] = x[o, j] (forward) or
    y[o, j] = x[o, pos[j]] (inverse).  Any dtype; the bytes are moved unchanged."""
    outer, rows, C = x.shape
    nb = rows // b
    xb = x.reshape(outer, nb, b, C)
    y = np.empty_like(xb)
    for j in range(nb):
        if inverse:
            y[:, j] = xb[:, int(pos[j])]
        else:
            y[:, int(pos[j])] = xb[:, j]
    return y.reshape(outer, rows, C)


# --------------------------------------------------------------------------------------------------
# communication-volume accounting (section 3.1: volume a rank must receive; section 3.2 and Figure 4:
# how widely a received block is shared by the rank's queries; section 3.3 and section 5.1 / Figure 9:
# relayed ring traffic versus demand-directed delivery)


def access_counts(mask: np.ndarray, nb: int) -> np.ndarray:
    """cnt[h][j] = number of the rank's local query rows whose mask selects block j (int64 [H][nb]).
    Written as the count itself: a loop over rows adding one per selected entry."""
    H, Lq = mask.shape[0], mask.shape[1]
    cnt = np.zeros((H, nb), dtype=np.int64)
    for h in range(H):
        for k in range(Lq):
            cnt[h] += np.asarray(mask[h, k, :nb]) != 0
    return cnt


def ring_distance(p: int, c: int, G: int) -> int:
    """Hops from producer p to consumer c along the ring p -> p+1 -> ... (section 2.3's Ring Attention)."""
    return (c - p) % G


def comm_volume(U_all: np.ndarray, placement: np.ndarray, G: int) -> dict:
    """Block counts of three ways to deliver every consumer's demand (one block = one head's K and V of b
    tokens).  U_all bool [G][H][nb]: consumer c's per-head demand union (Eq. 2 over c's own rows).

    direct [G][G]   direct[c][p] = |{(h, j) : P(j) = p, U_c[h][j]}| for c != p, 0 on the diagonal: each
                    selected block crosses one link, straight from its owner (section 5.1).
    relay  [G][G]   relay[p][k] = blocks of producer p on ring hop k (from p+k-1 to p+k), k = 1..G-1:
                    a block travels until its farthest consumer, each relay forwarding what ranks further
                    downstream still need (section 3.3; Figure 9(a): the first hop carries everything the
                    others selected); column 0 is 0.
    dense  [G]      dense[p] = (G-1) * H * |{j : P(j) = p}|: the whole shard of every head on every hop.
    """
    G_, H, nb = U_all.shape
    assert G_ == G
    P = [int(x) for x in np.asarray(placement).tolist()]
    direct = np.zeros((G, G), dtype=np.int64)
    relay = np.zeros((G, G), dtype=np.int64)
    dense = np.zeros(G, dtype=np.int64)
    for p in range(G):
        dense[p] = (G - 1) * H * sum(1 for j in range(nb) if P[j] == p)
    for h in range(H):
        for j in range(nb):
            p = P[j]
            far = 0
            for c in range(G):
                if c != p and U_all[c, h, j]:
                    direct[c, p] += 1
                    far = max(far, ring_distance(p, c, G))
            for k in range(1, far + 1):
                relay[p, k] += 1
    return dict(direct=direct, relay=relay, dense=dense)


def sharing_fractions(cnt: np.ndarray, placement: np.ndarray, r: int, Lq: int) -> np.ndarray:
    """Figure 4's quantity for rank r: for every remote block (h, j) the rank receives (P(j) != r and some
    local row selects it), the fraction of the rank's local query blocks that access it.  Returns the
    fractions as a float64 array (one entry per received remote block, in (h, j) order)."""
    P = np.asarray(placement)
    out = []
    H, nb = cnt.shape
    for h in range(H):
        for j in range(nb):
            if P[j] != r and cnt[h, j] > 0:
                out.append(cnt[h, j] / Lq)
    return np.array(out, dtype=np.float64)


# --------------------------------------------------------------------------------------------------
# mask materialisation from pooled tiles (section 4.2: block-sparse video DiT kernels build their block
# mask from pooled query and key tiles before the attention kernel runs; the evaluation uses CDF
# thresholds, and the Top-p rule with a Top-k safety floor comes from the FVAttn abstract on the pages)


def pool_blocks(X: np.ndarray, b: int, N: int, block_ids=None) -> np.ndarray:
    """Mean of the real token rows of every block: X uint16 (bf16 bits) [H][n*b][d] -> float64 [H][n][d].
    Block k covers rows k*b .. k*b+b-1 of X and is logical block block_ids[k] (default k), whose real
    tokens are those with index < N; padded rows are not counted."""
    H, rows, d = X.shape
    n = rows // b
    ids = np.arange(n) if block_ids is None else np.asarray(block_ids)
    x = bf16_to_f64(X)
    out = np.zeros((H, n, d))
    for k in range(n):
        real = min(b, N - int(ids[k]) * b)
        if real > 0:
            out[:, k] = x[:, k * b:k * b + real].sum(axis=1) / real
    return out


def block_scores(q_pooled: np.ndarray, k_pooled: np.ndarray, scale: float) -> np.ndarray:
    """s[h][k][j] = scale * <q_pooled[h][k], k_pooled[h][j]> (the block-level QK^T)."""
    return np.einsum("hkc,hjc->hkj", q_pooled, k_pooled) * scale


def select_row(scores: np.ndarray, tau: float, k_min: int) -> tuple[list, int]:
    """Top-p selection with a Top-k floor for one row of block scores.

    Blocks in descending score order (equal scores: ascending j); p_j = exp(s_j - max s) / Z; n_tau =
    the smallest n >= 1 whose first n blocks carry at least tau of the mass; n = min(nb, max(k_min,
    n_tau)).  Returns (the order, n): the selected blocks are order[:n]."""
    nb = len(scores)
    order = sorted(range(nb), key=lambda j: (-float(scores[j]), j))
    m = max(float(x) for x in scores)
    p = [np.exp(float(scores[j]) - m) for j in order]
    Z = float(sum(p))
    cum, n_tau = 0.0, nb
    for i in range(nb):
        cum += p[i]
        if cum >= tau * Z:
            n_tau = i + 1
            break
    return order, min(nb, max(k_min, n_tau))


def materialize_mask(q_pooled: np.ndarray, k_pooled: np.ndarray, scale: float, tau: float, k_min: int,
                     pitch: int) -> np.ndarray:
    """uint8 mask [H][Lq][pitch] (columns >= nb are 0) from pooled tiles: every row's selected blocks."""
    H, Lq, _ = q_pooled.shape
    nb = k_pooled.shape[1]
    s = block_scores(q_pooled, k_pooled, scale)
    mask = np.zeros((H, Lq, pitch), np.uint8)
    for h in range(H):
        for k in range(Lq):
            order, n = select_row(s[h, k], tau, k_min)
            mask[h, k, order[:n]] = 1
    return mask
