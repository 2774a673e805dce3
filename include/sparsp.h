/*
 * sparsp.h -- C ABI for one sequence-parallel rank's share of block-sparse attention on AMD Instinct
 * MI355X (gfx950).
 *
 * The operations follow "SparSP: Exploiting Communication Sparsity for Sequence-Parallel Video DiTs"
 * (full text, paperpeel.com page): a token sequence is cut into blocks of b tokens, every head h has a
 * block mask M[h, i, j] (query block i may attend to key block j), and a placement P assigns every block
 * to one of G sequence-parallel ranks.  For the queries of rank r the library computes
 *
 *   1. sparsp_local_query_blocks  -- Q_r = {i : P(i) = r}, ascending (section 4.1, Eq. 2).
 *   2. sparsp_demand_union        -- the per-head demand union of Eq. 2 (section 4.1) kept per head
 *                                    (section 5.2, head-preserving demand), and its compaction into
 *                                    packed slots enumerated by (source rank, head, block) in row-major
 *                                    order (section 5.2, metadata-free exchange).
 *   3. sparsp_pack_kv             -- the demanded K/V blocks copied into one compacted buffer whose
 *                                    per-source-rank segments are the payloads that would cross the
 *                                    link (sections 5.1 and 6.1), already in the attention kernel's
 *                                    layout (section 6.2 places arrived blocks into that layout).
 *   4. sparsp_block_sparse_attn   -- softmax(Q K^T / sqrt(d)) V (section 2.2) over the selected key
 *                                    blocks only, with an online softmax (section 2.3), reading K/V
 *                                    from the compacted buffer.
 *   5. sparsp_block_sparse_attn_segment, sparsp_merge_partial, sparsp_block_sparse_attn_segment_accumulate,
 *      sparsp_chunk_plan, sparsp_block_sparse_attn_chunk_accumulate
 *                                 -- the same attention restricted to one range of packed slots (one
 *                                    source rank's segment, consumed as it arrives: sections 5.1 and
 *                                    7), the log-sum-exp merge of such partial results (section 2.3's
 *                                    online softmax across pieces of KV), both fused in one call, and
 *                                    the consumption schedule of section 7: segments cut into head
 *                                    chunks, finer for the final remote segment (7.1), the chunk with the
 *                                    highest sparsity of a segment last (7.2).
 *   6. sparsp_placement_permutation, sparsp_permute_blocks
 *                                 -- the placement realised as a permutation of whole blocks into
 *                                    rank-major order, applied to hidden states and undone afterwards
 *                                    (section 4.3).
 *   7. sparsp_demand_counts, sparsp_comm_volume
 *                                 -- communication-volume accounting: how many local query blocks share
 *                                    each demanded block (section 3.2, Figure 4), and the blocks that
 *                                    demand-directed delivery, a relaying ring and a dense ring move
 *                                    (sections 3.1, 3.3 and 5.1, Figure 9).
 *   8. sparsp_pool_blocks, sparsp_materialize_mask
 *                                 -- the block mask itself, built from pooled query and key tiles
 *                                    (section 4.2): block means, block scores, and per row a Top-p
 *                                    (CDF threshold) selection with a Top-k floor.
 *
 * Conventions shared by every call
 *   - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 *   - Device pointers point to memory on the current HIP device and are owned by the caller.  The
 *     library allocates nothing, keeps no state between calls and never synchronises: work is enqueued
 *     on `stream` (a hipStream_t; NULL = the legacy default stream) in call order.
 *   - Arguments are checked before anything is launched; a failed check returns an error status and
 *     launches nothing.  Contents of device arrays (mask bytes, placement values) are not checked on
 *     the host; the kernels never read or write outside the documented extents even when they are
 *     inconsistent (out-of-range values are treated as "not selected").
 *   - SPARSP_ERR_HIP reports a launch failure; asynchronous device faults surface at the caller's next
 *     synchronisation.  sparsp_last_error() returns a message for the calling thread's last failure.
 *   - Every call is re-entrant and thread-safe.
 *
 * Geometry: nb = ceil(N / b) blocks; W = ceil(nb / 64) demand words per head.  Supported: d in {64, 128},
 * b in {64, 128}, 1 <= G <= 64, nb <= 16384, 0 <= Lq <= nb, H >= 1, 0 <= r < G.
 */
#ifndef SPARSP_H
#define SPARSP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSP_ABI_VERSION 7

typedef enum sparsp_status {
  SPARSP_OK = 0,
  SPARSP_ERR_INVALID = 1,      /* null pointer, bad size, stride or alignment                       */
  SPARSP_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels implement (d, b, G, nb limits)  */
  SPARSP_ERR_HIP = 3           /* the HIP runtime reported an error while launching                 */
} sparsp_status;

typedef struct sparsp_geometry {
  int32_t H;   /* heads                                                    */
  int32_t d;   /* head dimension (64 or 128)                               */
  int32_t b;   /* tokens per block (64 or 128)                             */
  int32_t N;   /* real tokens in the whole sequence (nb = ceil(N / b))      */
  int32_t G;   /* sequence-parallel ranks                                  */
  int32_t r;   /* the rank whose share is computed                         */
  int32_t Lq;  /* number of local query blocks, |Q_r|                      */
} sparsp_geometry;

/* ABI version (SPARSP_ABI_VERSION of the built library). */
int32_t sparsp_abi_version(void);

/* Static description of a status code. */
const char* sparsp_status_string(int32_t status);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char* sparsp_last_error(void);

/*
 * Q_r = {i : P(i) = r} in ascending order (section 4.1, Eq. 2; section 4.3 computes the placement once
 * per geometry, off the critical path).  HOST pointers.
 *   placement  [nb] int32, values in [0, G)           (read)
 *   q_blocks   [capacity] int32                        (written: the first *Lq entries)
 *   Lq         int32                                   (written: |Q_r|)
 * Errors: SPARSP_ERR_INVALID for null pointers, nb < 1, r outside [0, G), a placement value outside
 * [0, G), or capacity < |Q_r| (then nothing is written to q_blocks and *Lq holds the needed size).
 */
int32_t sparsp_local_query_blocks(const int32_t* placement, int32_t nb, int32_t G, int32_t r,
                                  int32_t* q_blocks, int32_t capacity, int32_t* Lq);

/*
 * Demand union and per-peer compaction (section 4.1 Eq. 2; section 5.2).  DEVICE pointers.
 *   mask         [H][Lq][mask_pitch] uint8, the rank's own rows M[h, i in Q_r (ascending), j];
 *                nonzero = selected; columns j >= nb are ignored.  mask_pitch >= nb, a multiple of 16,
 *                and mask 16-byte aligned.                                            (read)
 *   placement    [nb] int32, P(j) in [0, G)                                           (read)
 *   demand       [H][W] uint64: bit (j mod 64) of word (j / 64) = OR over local rows of M[h, ., j];
 *                bits >= nb are 0                                                      (written)
 *   seg_offsets  [G*H + 1] int32: first slot of (source rank p, head h) at index p*H + h,
 *                exclusive prefix sums of the counts; seg_offsets[G*H] = S, the total slot count
 *                                                                                      (written)
 *   slot_block   [H*nb] int32: logical block j of slot s, for s < S                   (written, s < S)
 *   slot_head    [H*nb] int32: head h of slot s, for s < S                            (written, s < S)
 *   slot_of      [H][nb] int32: slot of (h, j), or -1 if (h, j) is not demanded       (written)
 * Slots are numbered by source rank p = 0..G-1, then head h = 0..H-1, then ascending j with
 * P(j) = p, so the blocks owned by rank p form one contiguous range [seg_offsets[p*H], seg_offsets[(p+1)*H])
 * and each head inside it is contiguous.  The rank's own blocks (p = r) are included.  Results are
 * deterministic and bit-identical run to run.  slot_block and slot_head must hold H*nb entries (the
 * worst case), so S never has to be read on the host.
 * Errors: SPARSP_ERR_INVALID (null pointers, bad sizes, pitch or alignment);
 * SPARSP_ERR_UNSUPPORTED (G > 64, nb > 16384, or G*W*12 + (G*H+1)*4 bytes above 64 KiB).
 */
int32_t sparsp_demand_union(const sparsp_geometry* g, const uint8_t* mask, int64_t mask_pitch,
                            const int32_t* placement, uint64_t* demand, int32_t* seg_offsets,
                            int32_t* slot_block, int32_t* slot_head, int32_t* slot_of, void* stream);

/*
 * Pack the demanded K/V blocks into the compacted buffer (sections 5.1, 6.1, 6.2).  DEVICE pointers.
 *   K, V         [H][nb*b][d] bf16, token-major; rows >= N should be zero            (read)
 *   seg_offsets, slot_block, slot_head: as written by sparsp_demand_union            (read)
 *   slot_capacity  number of slots `packed` can hold (>= 1); slots s >= slot_capacity are not written
 *   packed       [slot_capacity][2][b*d] bf16.  Slot s = (h, j) = (slot_head[s], slot_block[s]) holds
 *                  part 0: K[h, j*b + t, c] at t*d + c        (the K block, token-major, b x d)
 *                  part 1: V[h, j*b + t, c] at c*b + t        (the V block transposed, d x b)
 *                for every s < min(S, slot_capacity); other slots are left untouched, and so is a slot
 *                whose slot_head or slot_block lies outside [0, H) or [0, nb)            (written)
 * Errors: SPARSP_ERR_INVALID (null pointers, slot_capacity < 1, misaligned K/V/packed: 16 bytes);
 * SPARSP_ERR_UNSUPPORTED (d or b outside {64, 128}).
 */
int32_t sparsp_pack_kv(const sparsp_geometry* g, const uint16_t* K, const uint16_t* V,
                       const int32_t* seg_offsets, const int32_t* slot_block, const int32_t* slot_head,
                       int32_t slot_capacity, uint16_t* packed, void* stream);

/*
 * Block-sparse flash attention for the local queries over the compacted K/V (sections 2.2, 2.3; Eq. 2's
 * mask).  DEVICE pointers.
 *   Q            [H][Lq*b][d] bf16: local query rows, blocks in Q_r order             (read)
 *   mask         as for sparsp_demand_union                                           (read)
 *   slot_of      [H][nb] int32 from sparsp_demand_union on the same mask              (read)
 *   packed       [slot_capacity][2][b*d] from sparsp_pack_kv                          (read)
 *   softmax_scale  multiplies Q K^T before the softmax (1/sqrt(d) for the paper's formula); finite, > 0
 *   O            [H][Lq*b][d] float32: softmax-weighted sum of V rows                  (written)
 *   lse          [H][Lq*b] float32: natural-log log-sum-exp of the scaled logits       (written)
 * For local block k of head h the keys are the real tokens (index < N) of every block j with
 * mask[h][k][j] != 0; key tokens of the last block at index >= N are excluded.  The blocks are visited in an
 * order chosen for L2 locality (at b = 128 each row starts at a column shared with its neighbouring query
 * blocks and wraps around); the result depends on the order only through rounding, and repeated calls on
 * the same inputs give the same bits.
 * A row with no key gives O = 0 and lse = -inf.  A selected block whose slot_of entry is negative or
 * >= slot_capacity is skipped.  Inputs are bf16; products accumulate in fp32 and the softmax
 * probabilities are rounded to bf16 before the P V product.
 * Errors: SPARSP_ERR_INVALID (null pointers, bad sizes, pitch, alignment, a scale that is not finite and > 0);
 * SPARSP_ERR_UNSUPPORTED (d or b outside {64, 128}, nb > 16384).
 */
int32_t sparsp_block_sparse_attn(const sparsp_geometry* g, const uint16_t* Q, const uint8_t* mask,
                                 int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                 int32_t slot_capacity, float softmax_scale, float* O, float* lse,
                                 void* stream);

/*
 * Block-sparse attention over the selected blocks whose slot lies in [slot_lo, slot_hi) only (sections 2.3,
 * 5.1 and 7: each source rank's segment of the payload is consumed as it arrives; segment p of rank r's
 * payload is [seg_offsets[p*H], seg_offsets[(p+1)*H]) as written by sparsp_demand_union).  DEVICE pointers;
 * arguments as for sparsp_block_sparse_attn, with packed holding at least slot_hi slots.
 *   O, lse       the partial result over those keys: softmax-weighted mean of their V rows and the
 *                log-sum-exp of their scaled logits; (0, -inf) for a row none of whose keys is in range
 * Errors: as for sparsp_block_sparse_attn; SPARSP_ERR_INVALID also when slot_lo < 0 or slot_hi < slot_lo.
 */
int32_t sparsp_block_sparse_attn_segment(const sparsp_geometry* g, const uint16_t* Q, const uint8_t* mask,
                                         int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                         int32_t slot_lo, int32_t slot_hi, float softmax_scale, float* O,
                                         float* lse, void* stream);

/*
 * sparsp_block_sparse_attn_segment and sparsp_merge_partial in one call (sections 2.3, 5.1 and 7): the
 * attention over the selected blocks whose slot lies in [slot_lo, slot_hi) is folded straight into the
 * running result instead of being written out and merged.  DEVICE pointers; arguments as for
 * sparsp_block_sparse_attn_segment, except
 *   O, lse       [H][Lq*b][d], [H][Lq*b] float32: the running result over the keys consumed so far (read,
 *                written); start from (0, -inf).  With lse_part and O_part the segment's result, lse <-
 *                ln(e^lse + e^lse_part) and O <- e^(lse_old - lse) O + e^(lse_part - lse) O_part.  Rows
 *                of a query block none of whose selected blocks lies in the range are not touched.
 * Calling it for every segment of the payload, in any order, gives the result of sparsp_block_sparse_attn
 * up to rounding.  Calls that update the same O and lse must be ordered (e.g. one stream).
 * Errors: as for sparsp_block_sparse_attn_segment.
 */
int32_t sparsp_block_sparse_attn_segment_accumulate(const sparsp_geometry* g, const uint16_t* Q, const uint8_t* mask,
                                                    int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                                    int32_t slot_lo, int32_t slot_hi, float softmax_scale, float* O,
                                                    float* lse, void* stream);

/*
 * One chunk of a consumption schedule (section 7): heads [h_lo, h_hi) of source rank p's segment, which are the
 * packed slots [slot_lo, slot_hi) (each head of a segment is contiguous), carrying `tiles` selected (head, local
 * query block, key block) triples of this rank's mask.
 */
typedef struct sparsp_chunk {
  int32_t p;
  int32_t h_lo, h_hi;
  int32_t slot_lo, slot_hi;
  int32_t reserved;  /* 0 */
  int64_t tiles;
} sparsp_chunk;

/*
 * The consumption schedule of the payload (section 7, Figure 11).  HOST pointers.  Segments are consumed in
 * ring order p = r, r+1, ..., r+G-1 (mod G): the local segment first and whole (section 7.1: it needs no
 * communication), every remote segment cut into `chunks_steady` head chunks except the final remote segment,
 * which is cut into `chunks_drain` (section 7.1: finer chunks where the pipeline drains).  A segment of c
 * chunks (c clamped to H) splits the heads into [floor(i*H/c), floor((i+1)*H/c)), i = 0..c-1.  Inside a
 * segment the chunks are ordered by decreasing tile count, ties by ascending h_lo, so the chunk with the
 * highest sparsity runs last (section 7.2).  Chunks without slots are left out.
 *   seg_offsets  [G*H + 1] int32, as written by sparsp_demand_union                              (read)
 *   counts       [H][nb] int32, as written by sparsp_demand_counts for the same mask             (read)
 *   placement    [nb] int32, P(j) in [0, G)                                                       (read)
 *   chunks       [capacity] sparsp_chunk: the schedule in execution order                         (written)
 *   n_chunks     number of chunks (written also when capacity is too small; at most G*H)
 * Folding every chunk with sparsp_block_sparse_attn_chunk_accumulate, in this order or any other, gives the
 * result of sparsp_block_sparse_attn up to rounding.
 * Errors: SPARSP_ERR_INVALID for null pointers, G outside [1, 64], H < 1, nb < 1, r outside [0, G), chunk
 * counts < 1, a placement value outside [0, G), decreasing seg_offsets, or capacity below the chunk count
 * (then nothing is written to chunks).
 */
int32_t sparsp_chunk_plan(const int32_t* seg_offsets, const int32_t* counts, const int32_t* placement, int32_t G,
                          int32_t H, int32_t nb, int32_t r, int32_t chunks_steady, int32_t chunks_drain,
                          sparsp_chunk* chunks, int32_t capacity, int32_t* n_chunks);

/*
 * sparsp_block_sparse_attn_segment_accumulate restricted to the heads [h_lo, h_hi): one chunk of a schedule
 * from sparsp_chunk_plan (section 7.2: attention is partitioned by heads).  Only that head range's (head,
 * local query block) items are launched; rows of other heads are not touched.  DEVICE pointers; arguments as
 * for sparsp_block_sparse_attn_segment_accumulate.
 * Errors: as for sparsp_block_sparse_attn_segment_accumulate; SPARSP_ERR_INVALID also unless
 * 0 <= h_lo <= h_hi <= H.
 */
int32_t sparsp_block_sparse_attn_chunk_accumulate(const sparsp_geometry* g, const uint16_t* Q, const uint8_t* mask,
                                                  int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                                  int32_t slot_lo, int32_t slot_hi, int32_t h_lo, int32_t h_hi,
                                                  float softmax_scale, float* O, float* lse, void* stream);

/*
 * Fold a partial attention result over one key set into a running result over a disjoint key set (section
 * 2.3, online softmax across pieces of KV).  DEVICE pointers, rows = H * Lq * b of d floats:
 *   O, lse            [H][Lq*b][d], [H][Lq*b] float32: the running result                (read, written)
 *   O_part, lse_part  the partial result, e.g. from sparsp_block_sparse_attn_segment     (read)
 * With m = max(lse, lse_part): lse <- m + ln(e^(lse - m) + e^(lse_part - m)) and
 * O <- e^(lse_old - lse) O + e^(lse_part - lse) O_part; a row where both are -inf stays (0, -inf), so a
 * running result may start as (0, -inf).  Merging every segment of the payload, in any order, gives the
 * result of sparsp_block_sparse_attn up to rounding: each piece rounds its probabilities to bf16 relative
 * to its own running maximum.
 * Errors: SPARSP_ERR_INVALID (null pointers, O or O_part not 16-byte aligned); SPARSP_ERR_UNSUPPORTED (d).
 */
int32_t sparsp_merge_partial(const sparsp_geometry* g, float* O, float* lse, const float* O_part,
                             const float* lse_part, void* stream);

/*
 * The placement as a permutation of whole blocks (section 4.3: the placement is computed once per model
 * geometry and SP degree as a deterministic map from logical blocks to (rank, offset) pairs).  HOST
 * pointers.  Rank-major order: rank 0's blocks first, then rank 1's, ...; inside a rank, ascending logical
 * index, so rank p's range of the permuted sequence holds Q_p in the order every other call uses.
 *   placement     [nb] int32, P(j) in [0, G)                                               (read)
 *   pos           [nb] int32: the permuted position of logical block j                    (written)
 *   rank_offsets  [G + 1] int32: rank p's blocks occupy [rank_offsets[p], rank_offsets[p + 1]);
 *                 rank_offsets[G] = nb                                                      (written)
 * Errors: SPARSP_ERR_INVALID for null pointers, nb < 1, G < 1, or a placement value outside [0, G) (then
 * nothing is written).
 */
int32_t sparsp_placement_permutation(const int32_t* placement, int32_t nb, int32_t G, int32_t* pos,
                                     int32_t* rank_offsets);

/*
 * Apply the block permutation to a tensor (section 4.3: hidden states and position-dependent data are
 * permuted before the distributed region; the inverse restores the original token order after it).
 * DEVICE pointers.  The tensor is `outer` independent sequences of nb blocks of block_bytes bytes each
 * (e.g. hidden states [nb*b][C] with outer = 1 and block_bytes = b*C*element size, or per-head
 * [H][nb*b][d] with outer = H and block_bytes = b*d*element size).
 *   src      [outer][nb][block_bytes]                                                      (read)
 *   dst      [outer][nb][block_bytes]; must not overlap src                                (written)
 *   pos      [nb] int32, a permutation of 0..nb-1 (from sparsp_placement_permutation)     (read)
 *   inverse  0: dst[o][pos[j]] = src[o][j];  1: dst[o][j] = src[o][pos[j]]
 * Bytes are moved unchanged.  A pos entry outside [0, nb) moves nothing for that block (its contents are
 * not checked on the host).
 * Errors: SPARSP_ERR_INVALID (null pointers, outer < 0, nb < 1, block_bytes not a positive multiple of 16,
 * src or dst not 16-byte aligned, src == dst); SPARSP_ERR_UNSUPPORTED (more than 2^31 - 1 workgroups).
 */
int32_t sparsp_permute_blocks(const void* src, void* dst, int64_t outer, int32_t nb, int64_t block_bytes,
                              const int32_t* pos, int32_t inverse, void* stream);

/*
 * Access counts of the rank's mask rows (section 3.2 and Figure 4: the share of a rank's query blocks that
 * use each KV block it receives).  DEVICE pointers.
 *   mask     as for sparsp_demand_union                                                    (read)
 *   counts   [H][nb] int32: number of local rows k with mask[h][k][j] != 0                 (written)
 * counts > 0 is the demand union of sparsp_demand_union.  Deterministic, integer-only.
 * Errors: as for sparsp_demand_union's geometry and mask checks; SPARSP_ERR_INVALID for a NULL counts.
 */
int32_t sparsp_demand_counts(const sparsp_geometry* g, const uint8_t* mask, int64_t mask_pitch, int32_t* counts,
                             void* stream);

/*
 * Communication volume of delivering every rank's demand, in blocks (one block = one head's K and V of b
 * tokens; multiply by 2*b*d*element size for bytes).  HOST pointers.  Sections 3.1 and 3.3, section 5.1 and
 * Figure 9.
 *   demand     [G][H][W] uint64: demand[c] is consumer c's union as written by sparsp_demand_union for
 *              geometry r = c (bits >= nb are ignored)                                      (read)
 *   placement  [nb] int32, P(j) in [0, G)                                                   (read)
 *   direct     [G][G] int64: direct[c][p] = blocks of producer p that consumer c demands, c != p; the
 *              diagonal is 0 (demand-directed delivery: each block crosses one link once)  (written)
 *   relay      [G][G] int64: relay[p][k] = blocks of producer p on ring hop k (from rank p+k-1 to p+k),
 *              k = 1..G-1, when each rank passes on what ranks further along still demand; column 0 is 0
 *                                                                                            (written)
 *   dense      [G] int64: (G-1)*H*|{j : P(j) = p}|, the whole shard on every hop            (written)
 * Errors: SPARSP_ERR_INVALID for null pointers, G outside [1, 64], H < 1, nb < 1, or a placement value
 * outside [0, G) (then nothing is written).
 */
int32_t sparsp_comm_volume(const uint64_t* demand, int32_t G, int32_t H, int32_t nb, const int32_t* placement,
                           int64_t* direct, int64_t* relay, int64_t* dense);

/*
 * Block-mean pooling (section 4.2: masks are materialised from pooled query and key tiles).  DEVICE
 * pointers.
 *   X          [H][n_blocks*b][d] bf16: n_blocks blocks of b token rows per head         (read)
 *   block_ids  [n_blocks] int32: logical block id of block k, which fixes its real rows (tokens < N);
 *              NULL means block k is logical block k (all of K: n_blocks = nb; for the local queries
 *              pass q_blocks)                                                              (read)
 *   pooled     [H][n_blocks][d] float32: mean of the block's real rows, 0 if it has none   (written)
 * Rows at token index >= N are not read.  Sums are fp32 in a fixed order (deterministic).
 * Errors: SPARSP_ERR_INVALID (null pointers, n_blocks outside [0, nb], X or pooled not 16-byte aligned);
 * SPARSP_ERR_UNSUPPORTED (d or b outside {64, 128}, H > 65535).
 */
int32_t sparsp_pool_blocks(const sparsp_geometry* g, const uint16_t* X, int32_t n_blocks, const int32_t* block_ids,
                           float* pooled, void* stream);

/*
 * Block mask of the rank's rows from pooled tiles (section 4.2).  DEVICE pointers.
 *   q_pooled   [H][Lq][d] float32: pooled local query blocks (sparsp_pool_blocks over Q)   (read)
 *   k_pooled   [H][nb][d] float32: pooled key blocks (sparsp_pool_blocks over K)           (read)
 *   softmax_scale  multiplies the pooled dot products (1/sqrt(d)); finite, > 0
 *   tau        CDF threshold in [0, 1]
 *   k_min      Top-k floor, >= 0
 *   mask       [H][Lq][mask_pitch] uint8, the format sparsp_demand_union and sparsp_block_sparse_attn
 *              read: 1 for a selected block, 0 elsewhere, columns >= nb included         (written)
 * Row k of head h: scores s_j = softmax_scale * <q_pooled[h][k], k_pooled[h][j]>; blocks in descending
 * score order (equal scores: ascending j); weights exp(s_j - max s); the first n blocks are selected,
 * n = min(nb, max(k_min, n_tau)) with n_tau the shortest prefix holding at least tau of the total weight.
 * Arithmetic is fp32: a block whose score or prefix weight sits within rounding of the decision may
 * fall either way.
 * Errors: SPARSP_ERR_INVALID (null pointers, bad pitch or alignment, tau outside [0, 1], k_min < 0, a
 * scale that is not finite and > 0); SPARSP_ERR_UNSUPPORTED (d or b outside {64, 128}, nb > 16384,
 * H > 65535).
 */
int32_t sparsp_materialize_mask(const sparsp_geometry* g, const float* q_pooled, const float* k_pooled,
                                float softmax_scale, float tau, int32_t k_min, uint8_t* mask, int64_t mask_pitch,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSP_H */
