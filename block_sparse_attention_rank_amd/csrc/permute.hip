// Placement permutation of whole blocks (SparSP paper, section 4.3: the dependency-aware placement is
// realised as one fixed permutation of logical blocks to (rank, offset) order, applied to the hidden
// states before the distributed region and inverted after it; blocks move whole, so their contents and
// membership are unchanged).
//
// The copy is HBM-bound: every byte is read once and written once with 16-byte vector accesses.  A
// workgroup of 256 threads moves a power-of-two group of blocks (small blocks) or a 16 KiB chunk of one
// block (large blocks); consecutive lanes touch consecutive 16-byte vectors of the same block, and each
// thread issues all its loads before its stores.
#include "sparsp_internal.h"

namespace sparsp {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kPermThreads = 256;
constexpr int kPermVec = 4;  // 16-byte vectors per thread

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                               const int32_t* __restrict__ pos, int64_t blocks,
                                                               int nb, int64_t block_vecs, int tpb_log2, int chunks,
                                                               int inverse) {
  const int tpb = 1 << tpb_log2;  // threads per block
  const int bpw = kPermThreads >> tpb_log2;
  const int g = threadIdx.x >> tpb_log2, lt = threadIdx.x & (tpb - 1);
  const int c = blockIdx.x % chunks;
  const int64_t blk = (int64_t)(blockIdx.x / chunks) * bpw + g;  // (outer, logical block) index
  if (blk >= blocks) return;
  const int64_t o = blk / nb;
  const int j = (int)(blk - o * nb);
  const int p = pos[j];
  if (p < 0 || p >= nb) return;  // not a permutation entry: nothing is moved for this block
  const int sj = inverse ? p : j, dj = inverse ? j : p;
  const u32x4* s = src + (o * nb + sj) * block_vecs;
  u32x4* d = dst + (o * nb + dj) * block_vecs;
  const int64_t v0 = (int64_t)c * tpb * kPermVec + lt;
  u32x4 v[kPermVec];
#pragma unroll
  for (int i = 0; i < kPermVec; ++i) {
    const int64_t idx = v0 + (int64_t)i * tpb;
    if (idx < block_vecs) v[i] = s[idx];
  }
#pragma unroll
  for (int i = 0; i < kPermVec; ++i) {
    const int64_t idx = v0 + (int64_t)i * tpb;
    if (idx < block_vecs) d[idx] = v[i];
  }
}

}  // namespace

hipError_t launch_permute(const void* src, void* dst, int64_t outer, int nb, int64_t block_bytes, const int32_t* pos,
                          int inverse, hipStream_t stream) {
  const int64_t block_vecs = block_bytes / 16;
  const int64_t blocks = outer * nb;
  if (blocks == 0 || block_vecs == 0) return hipSuccess;
  // Threads per block: the smallest power of two >= block_vecs / kPermVec, between 16 and 256.
  int tpb_log2 = 4;
  while (tpb_log2 < 8 && ((int64_t)kPermVec << tpb_log2) < block_vecs) ++tpb_log2;
  const int64_t per_wg = (int64_t)kPermVec << tpb_log2;
  const int64_t chunks = (block_vecs + per_wg - 1) / per_wg;
  const int64_t bpw = kPermThreads >> tpb_log2;
  const int64_t grid = (blocks + bpw - 1) / bpw * chunks;
  if (grid > 0x7fffffffll || chunks > 0x7fffffffll) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)grid), dim3(kPermThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), pos, blocks, nb, block_vecs,
                     tpb_log2, (int)chunks, inverse);
  return hipGetLastError();
}

}  // namespace sparsp
