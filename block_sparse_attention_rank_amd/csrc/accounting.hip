// Per-block access counts of one rank's mask rows: cnt[h][j] = number of the rank's local query blocks
// whose row selects key block j.  SparSP paper, section 3.2 and Figure 4: how many of a rank's queries
// share each received block is what decides how much a placement wastes; the count is also Eq. 2's
// demand union (cnt > 0) with multiplicity.
//
// Same streaming shape as the union: each thread walks 16-byte vectors down one column group (rows
// strided by 16), turns every byte into 0/1 with shifts inside its 32-bit word, keeps 16 column counters,
// and the 16 row groups are summed through LDS.  Integer-only and deterministic.
#include "sparsp_internal.h"

namespace sparsp {
namespace {

constexpr int kCountThreads = 256;
constexpr int kCountCols = 256;       // mask columns per workgroup
constexpr int kCountColGroups = 16;   // 16-byte column groups per row
constexpr int kCountRowGroups = kCountThreads / kCountColGroups;

// Bit 8k of the result is 1 when byte k of w is nonzero (the OR of its eight bits folded down).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
  w |= w >> 4;
  w |= w >> 2;
  w |= w >> 1;
  return w & 0x01010101u;
}

__global__ __launch_bounds__(kCountThreads) void counts_kernel(const uint8_t* __restrict__ mask, int64_t pitch, int Lq,
                                                               int nb, int32_t* __restrict__ counts) {
  __shared__ int part[kCountRowGroups][kCountCols];

  const int h = blockIdx.y;
  const int col0 = blockIdx.x * kCountCols;
  const int t = threadIdx.x;
  const int cg = t % kCountColGroups, rg = t / kCountColGroups;
  const int col = col0 + cg * 16;

  int c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = 0;
  if (col < pitch) {  // pitch is a multiple of 16, so the whole vector lies inside the row
    const uint8_t* p = mask + (int64_t)h * Lq * pitch + col;
    for (int row = rg; row < Lq; row += kCountRowGroups) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + (int64_t)row * pitch);
      const uint32_t w[4] = {nonzero_bytes(v.x), nonzero_bytes(v.y), nonzero_bytes(v.z), nonzero_bytes(v.w)};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) c[4 * q + k] += (w[q] >> (8 * k)) & 1u;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) part[rg][cg * 16 + i] = c[i];
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int r = 0; r < kCountRowGroups; ++r) s += part[r][t];
  if (col0 + t < nb) counts[(int64_t)h * nb + col0 + t] = s;
}

}  // namespace

hipError_t launch_counts(const Dims& g, const uint8_t* mask, int64_t pitch, int32_t* counts, hipStream_t stream) {
  const dim3 grid((unsigned)((g.nb + kCountCols - 1) / kCountCols), (unsigned)g.H);
  hipLaunchKernelGGL(counts_kernel, grid, dim3(kCountThreads), 0, stream, mask, pitch, g.Lq, g.nb, counts);
  return hipGetLastError();
}

}  // namespace sparsp
