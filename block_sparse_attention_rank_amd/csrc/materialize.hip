// Block-mask materialisation from pooled tiles (SparSP paper, section 4.2: the block-sparse video DiT
// kernels it targets build their mask from pooled query and key tiles before attention starts; receivers
// combine remote key summaries with local query summaries and materialise the demand on the GPU).
//
// pool_kernel: mean of the real token rows of each block of b rows (one workgroup per (head, block);
// 16-byte loads, fp32 sums, row groups combined through LDS in a fixed order).  HBM-bound: it reads
// every token of K once.
//
// select_kernel: one workgroup per (head, local query block).  Block scores s_j = scale <q, k_j> against
// every pooled key; the (score, block) pairs are sorted in LDS by a bitonic network into descending
// score order (equal scores: ascending block); the softmax weights exp(s - max) are prefix-summed in
// that order; the row keeps the smallest prefix holding at least tau of the mass, but at least k_min
// blocks (a Top-p rule with a Top-k floor), and writes the uint8 mask row the demand union and the
// attention consume.
#include <math.h>

#include "sparsp_internal.h"

namespace sparsp {
namespace {

constexpr int kPoolThreads = 256;

template <int D, int B>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const uint16_t* __restrict__ X, int n_blocks,
                                                            const int32_t* __restrict__ block_ids, int N,
                                                            float* __restrict__ pooled) {
  constexpr int CV = D / 8;                 // 16-byte column vectors per row
  constexpr int RG = kPoolThreads / CV;     // row groups
  __shared__ float part[RG][D];

  const int k = blockIdx.x, h = blockIdx.y;
  const int t = threadIdx.x, cv = t % CV, rg = t / CV;
  const int id = block_ids ? block_ids[k] : k;
  const int real = min(B, N - id * B);  // real token rows of this block (<= 0: none)
  const uint16_t* base = X + ((int64_t)h * n_blocks + k) * B * D + cv * 8;

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int row = rg; row < real; row += RG) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)row * D);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += __uint_as_float(w[q] << 16);               // bf16 -> fp32 is exact
      acc[2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rg][cv * 8 + i] = acc[i];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) s += part[r][t];
    pooled[((int64_t)h * n_blocks + k) * D + t] = real > 0 ? s / (float)real : 0.f;
  }
}

// Monotone map of a float to an unsigned key (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// NT threads: 256 for rows of up to 1024 blocks, 1024 above (the sort's passes are separated by barriers,
// so more threads per row shorten every pass).
template <int D, int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                                int Lq, int nb, int np2, float scale, float tau,
                                                                int k_min, uint8_t* __restrict__ mask, int64_t pitch) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);        // [np2]
  float* cum = reinterpret_cast<float*>(keys + np2);          // [np2]
  float* qv = cum + np2;                                      // [D]
  int* wsum = reinterpret_cast<int*>(qv + D);                 // scan scratch: one entry per wave (<= 16)
  uint8_t* sel = reinterpret_cast<uint8_t*>(wsum + 16);       // [pitch]

  const int k = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  if (t < D) qv[t] = qp[((int64_t)h * Lq + k) * D + t];
  __syncthreads();

  // Scores, keyed so that an ascending sort gives descending score and, among equal scores, ascending j.
  const float4* kh = reinterpret_cast<const float4*>(kp + (int64_t)h * nb * D);
  for (int j = t; j < np2; j += NT) {
    uint64_t key = ~0ull;
    if (j < nb) {
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < D / 4; ++c) {
        const float4 kv = kh[(int64_t)j * (D / 4) + c];
        s += qv[4 * c] * kv.x + qv[4 * c + 1] * kv.y + qv[4 * c + 2] * kv.z + qv[4 * c + 3] * kv.w;
      }
      key = ((uint64_t)(~ordered_bits(s * scale)) << 32) | (uint32_t)j;
    }
    keys[j] = key;
  }
  for (int i = t; i < pitch; i += NT) sel[i] = 0;
  __syncthreads();

  // Bitonic sort, ascending, of np2 keys (np2 a power of two); every thread takes whole compare pairs.
  // A pass of stride s < 64 keeps each wave inside its own 128-key chunks (pair q of a wave's 64 maps into
  // chunk q / 64), so the passes of stride 32 .. 1 of one merge size run back to back without a workgroup
  // barrier: a wave's LDS accesses complete in order.  Larger strides cross waves and end in a barrier.
  auto pass = [&](int size, int stride) {
    for (int q = t; q < np2 / 2; q += NT) {
      const int i = ((q & ~(stride - 1)) << 1) | (q & (stride - 1));
      const int p = i + stride;
      const uint64_t a = keys[i], b = keys[p];
      const bool up = (i & size) == 0;
      if ((a > b) == up) {
        keys[i] = b;
        keys[p] = a;
      }
    }
  };
  for (int size = 2; size <= np2; size <<= 1) {
    int stride = size >> 1;
    for (; stride >= 64; stride >>= 1) {
      pass(size, stride);
      __syncthreads();
    }
    for (; stride > 0; stride >>= 1) pass(size, stride);
    __syncthreads();
  }

  // Softmax weights in sorted order and their inclusive prefix sums.  Each thread scans a run of
  // consecutive entries; the runs' totals are scanned across the workgroup in thread order.
  const float smax = from_ordered_bits(~(uint32_t)(keys[0] >> 32));
  const int per = (np2 + NT - 1) / NT;
  const int i0 = t * per;
  float run = 0.f;
  for (int i = i0; i < min(i0 + per, nb); ++i) {
    run += expf(from_ordered_bits(~(uint32_t)(keys[i] >> 32)) - smax);
    cum[i] = run;
  }
  // exclusive scan of the run totals: within the wave by shuffles, then across the waves through LDS
  const int lane = t % 64, wave = t / 64;
  float incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  float* wtot = reinterpret_cast<float*>(wsum);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  float base = incl - run;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  for (int i = i0; i < min(i0 + per, nb); ++i) cum[i] += base;
  __syncthreads();

  // n_tau = 1 + the number of prefixes still short of tau of the total mass (cum is nondecreasing).
  const float target = tau * cum[nb - 1];
  int below = 0;
  for (int i = t; i < nb; i += NT) below += cum[i] < target ? 1 : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) below += __shfl_xor(below, off, 64);
  __syncthreads();
  if (lane == 0) wsum[wave] = below;
  __syncthreads();
  int n_tau = 1;
  for (int w = 0; w < NT / 64; ++w) n_tau += wsum[w];
  const int n = min(nb, max(k_min, n_tau));

  for (int i = t; i < n; i += NT) sel[(uint32_t)keys[i]] = 1;
  __syncthreads();
  uint8_t* row = mask + ((int64_t)h * Lq + k) * pitch;
  for (int i = t * 16; i < pitch; i += NT * 16)
    *reinterpret_cast<uint4*>(row + i) = *reinterpret_cast<const uint4*>(sel + i);
}

template <int D>
hipError_t launch_pool_d(const Dims& g, const uint16_t* X, int n_blocks, const int32_t* block_ids, float* pooled,
                         hipStream_t stream) {
  const dim3 grid((unsigned)n_blocks, (unsigned)g.H);
  if (g.b == 128)
    hipLaunchKernelGGL((pool_kernel<D, 128>), grid, dim3(kPoolThreads), 0, stream, X, n_blocks, block_ids, g.N, pooled);
  else
    hipLaunchKernelGGL((pool_kernel<D, 64>), grid, dim3(kPoolThreads), 0, stream, X, n_blocks, block_ids, g.N, pooled);
  return hipGetLastError();
}

}  // namespace

// Sort size: a power of two >= nb, at least 4 so that the selection bytes start 16-byte aligned.
size_t select_lds_bytes(int nb, int d, int64_t pitch) {
  int np2 = 4;
  while (np2 < nb) np2 <<= 1;
  return (size_t)np2 * 12 + (size_t)d * 4 + 64 + (size_t)pitch;
}

hipError_t launch_pool(const Dims& g, const uint16_t* X, int n_blocks, const int32_t* block_ids, float* pooled,
                       hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  return g.d == 128 ? launch_pool_d<128>(g, X, n_blocks, block_ids, pooled, stream)
                    : launch_pool_d<64>(g, X, n_blocks, block_ids, pooled, stream);
}

hipError_t launch_select(const Dims& g, const float* q_pooled, const float* k_pooled, float scale, float tau,
                         int k_min, uint8_t* mask, int64_t pitch, hipStream_t stream) {
  if (g.Lq == 0) return hipSuccess;
  int np2 = 4;
  while (np2 < g.nb) np2 <<= 1;
  const size_t lds = select_lds_bytes(g.nb, g.d, pitch);
  const dim3 grid((unsigned)g.Lq, (unsigned)g.H);
  const bool wide = np2 > 1024;
  if (g.d == 128 && wide)
    hipLaunchKernelGGL((select_kernel<128, 1024>), grid, dim3(1024), lds, stream, q_pooled, k_pooled, g.Lq, g.nb,
                       np2, scale, tau, k_min, mask, pitch);
  else if (g.d == 128)
    hipLaunchKernelGGL((select_kernel<128, 256>), grid, dim3(256), lds, stream, q_pooled, k_pooled, g.Lq, g.nb, np2,
                       scale, tau, k_min, mask, pitch);
  else if (wide)
    hipLaunchKernelGGL((select_kernel<64, 1024>), grid, dim3(1024), lds, stream, q_pooled, k_pooled, g.Lq, g.nb,
                       np2, scale, tau, k_min, mask, pitch);
  else
    hipLaunchKernelGGL((select_kernel<64, 256>), grid, dim3(256), lds, stream, q_pooled, k_pooled, g.Lq, g.nb, np2,
                       scale, tau, k_min, mask, pitch);
  return hipGetLastError();
}

}  // namespace sparsp
