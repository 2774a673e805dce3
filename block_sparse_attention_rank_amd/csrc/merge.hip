// Merge of two partial attention results over disjoint key sets (SparSP paper, section 2.3: attention
// consumes KV piece by piece with an online softmax; section 5.1: the payload arrives one source rank at a
// time).  A partial result is (O, lse): the softmax-weighted mean of the V rows of its keys and the
// natural-log log-sum-exp of their scaled logits; an empty key set is (0, -inf).  For two parts a and b,
// with m = max(lse_a, lse_b):
//   lse = m + ln(e^(lse_a - m) + e^(lse_b - m)),   O = (e^(lse_a - lse) O_a + e^(lse_b - lse) O_b).
// The kernel is elementwise and HBM-bound: it reads O, O_part and both lse rows and rewrites O and lse.
#include <math.h>

#include "sparsp_internal.h"

namespace sparsp {
namespace {

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(int64_t rows, float* __restrict__ O,
                                                              float* __restrict__ lse,
                                                              const float* __restrict__ O_part,
                                                              const float* __restrict__ lse_part) {
  constexpr int kChunks = D / 4;                      // float4 chunks per row
  constexpr int kRows = kMergeThreads / kChunks;      // rows per workgroup
  const int64_t r = (int64_t)blockIdx.x * kRows + threadIdx.x / kChunks;
  const int c = threadIdx.x % kChunks;
  float lse_new = -INFINITY;
  if (r < rows) {
    const float a = lse[r], b = lse_part[r];
    const float m = fmaxf(a, b);
    if (m != -INFINITY) {  // both -inf: both parts empty, O stays 0
      constexpr float kLog2e = 1.4426950408889634f;
      const float wa = __builtin_amdgcn_exp2f((a - m) * kLog2e), wb = __builtin_amdgcn_exp2f((b - m) * kLog2e);
      const float inv = 1.f / (wa + wb);
      lse_new = m + logf(wa + wb);
      float4* o = reinterpret_cast<float4*>(O + r * D) + c;
      const float4 x = *o, y = reinterpret_cast<const float4*>(O_part + r * D)[c];
      const float fa = wa * inv, fb = wb * inv;
      *o = make_float4(fa * x.x + fb * y.x, fa * x.y + fb * y.y, fa * x.z + fb * y.z, fa * x.w + fb * y.w);
    }
  }
  __syncthreads();  // every thread of the row has read the old lse
  if (r < rows && c == 0) lse[r] = lse_new;
}

}  // namespace

hipError_t launch_merge(int64_t rows, int d, float* O, float* lse, const float* O_part, const float* lse_part,
                        hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int rows_per_wg = kMergeThreads / (d / 4);
  const unsigned grid = (unsigned)((rows + rows_per_wg - 1) / rows_per_wg);
  if (d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kMergeThreads), 0, stream, rows, O, lse, O_part, lse_part);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kMergeThreads), 0, stream, rows, O, lse, O_part, lse_part);
  return hipGetLastError();
}

}  // namespace sparsp
