// Internal declarations shared by the HIP translation units of libsparsp (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparsp {

// Sizes derived from the public geometry after validation.
struct Dims {
  int H, d, b, N, G, r, Lq;
  int nb;  // ceil(N / b)
  int W;   // ceil(nb / 64)
};

constexpr int kMaxRanks = 64;
constexpr int kMaxBlocks = 16384;
constexpr int kCompactLdsLimit = 64 * 1024;

inline size_t compact_lds_bytes(const Dims& g) {
  return (size_t)g.G * g.W * 12 + ((size_t)g.G * g.H + 1) * 4;
}

hipError_t launch_union(const Dims& g, const uint8_t* mask, int64_t pitch, uint64_t* demand,
                        hipStream_t stream);
hipError_t launch_compact(const Dims& g, const int32_t* placement, const uint64_t* demand,
                          int32_t* seg_offsets, int32_t* slot_block, int32_t* slot_head,
                          int32_t* slot_of, hipStream_t stream);
hipError_t launch_pack(const Dims& g, const uint16_t* K, const uint16_t* V, const int32_t* seg_offsets,
                       const int32_t* slot_block, const int32_t* slot_head, int32_t slot_capacity,
                       uint16_t* packed, hipStream_t stream);
// Attention of heads [h_lo, h_hi) over the selected blocks whose slot lies in [slot_lo, slot_hi); only those
// heads' (head, query block) items are launched.  accumulate = 0 writes (O, lse); 1 folds the result into the
// running (O, lse) by their log-sum-exp (rows without keys in range untouched).  anchored = 1 (the single-pass
// call) walks each row's blocks from the anchor column of its group of query blocks instead of from the first.
hipError_t launch_attention(const Dims& g, const uint16_t* Q, const uint8_t* mask, int64_t pitch,
                            const int32_t* slot_of, const uint16_t* packed, int32_t slot_lo, int32_t slot_hi,
                            int32_t h_lo, int32_t h_hi, float softmax_scale, float* O, float* lse, int accumulate,
                            int anchored, hipStream_t stream);
// Fold a partial (O_part, lse_part) into (O, lse), rows of d floats.
hipError_t launch_merge(int64_t rows, int d, float* O, float* lse, const float* O_part, const float* lse_part,
                        hipStream_t stream);

// cnt[h][j] = number of the rank's mask rows of head h that select block j.
hipError_t launch_counts(const Dims& g, const uint8_t* mask, int64_t pitch, int32_t* counts, hipStream_t stream);

// Block means of the real rows: X [H][n_blocks*b][d] bf16 -> pooled [H][n_blocks][d] fp32; block k is logical
// block block_ids[k] (k when block_ids is null).
hipError_t launch_pool(const Dims& g, const uint16_t* X, int n_blocks, const int32_t* block_ids, float* pooled,
                       hipStream_t stream);
// Mask rows [H][Lq][pitch] from pooled tiles: Top-p (tau) with a Top-k floor (k_min) over the block scores.
hipError_t launch_select(const Dims& g, const float* q_pooled, const float* k_pooled, float scale, float tau,
                         int k_min, uint8_t* mask, int64_t pitch, hipStream_t stream);
constexpr int kMaxSelectBlocks = kMaxBlocks;

// Move whole blocks: dst[o][pos[j]] = src[o][j] (inverse = 0) or dst[o][j] = src[o][pos[j]] (inverse = 1).
hipError_t launch_permute(const void* src, void* dst, int64_t outer, int nb, int64_t block_bytes, const int32_t* pos,
                          int inverse, hipStream_t stream);

// Number of XCDs whose L2 slices a launch is spread over (MI355X: 8).  Workgroup ids are handed to the
// XCDs round-robin, so kernels that want neighbouring work items to share an L2 remap their ids.
constexpr int kXcds = 8;

// Items dealt to the XCDs in chunks of `Chunk` consecutive items, cyclically: XCD x runs chunks x, x + 8,
// x + 16, ... in order.  Neighbouring items (neighbouring query blocks of one head) stay on one XCD and
// share its L2, while every XCD samples all heads, which balances heads of different cost.  Valid for a
// grid of a multiple of 8 * Chunk workgroups; ids past the real item count are returned as they are
// (callers skip them).
template <int Chunk>
__device__ __forceinline__ int xcd_chunked(int pid) {
  const int xcd = pid % kXcds, idx = pid / kXcds;
  return ((idx / Chunk) * kXcds + xcd) * Chunk + idx % Chunk;
}

__device__ __forceinline__ int xcd_remap(int pid, int total) {
  const int xcd = pid % kXcds, idx = pid / kXcds;
  const int base = total / kXcds, rem = total % kXcds;
  const int start = xcd < rem ? xcd * (base + 1) : rem * (base + 1) + (xcd - rem) * base;
  return start + idx;
}

}  // namespace sparsp
