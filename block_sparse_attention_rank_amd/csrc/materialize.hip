// Block-mask materialisation from pooled tiles (SparSP paper, section 4.2: the block-sparse video DiT
// kernels it targets build their mask from pooled query and key tiles before attention starts; receivers
// combine remote key summaries with local query summaries and materialise the demand on the GPU).
//
// pool_kernel: mean of the real token rows of each block of b rows (one workgroup per (head, block);
// 16-byte loads, fp32 sums, row groups combined through LDS in a fixed order).  HBM-bound: it reads
// every token of K once.
//
// select_kernel: one workgroup per (head, local query block); every thread keeps up to four of the row's
// blocks in registers.  Block scores s_j = scale <q, k_j> against every pooled key are keyed so that
// ascending key order is descending score (equal scores: ascending block); the softmax weights exp(s - max)
// are summed, and the smallest key threshold whose blocks hold at least tau of the weight is found bit by
// bit with workgroup reductions in a fixed order (no sort); a second, count-only search applies the Top-k
// floor k_min.  The row keeps the blocks at or below the threshold (a Top-p rule with a Top-k floor) and
// writes the uint8 mask row the demand union and the attention consume.  Integer counts and fixed-order
// fp32 sums make the result deterministic.
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

// 64-bit lane exchange: the value of lane (this lane ^ m).
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const unsigned lo = (unsigned)__shfl_xor((int)(uint32_t)v, m, 64);
  const unsigned hi = (unsigned)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Monotone map of a float to an unsigned key (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// NT threads: 256 for rows of up to 1024 blocks, 1024 above; each thread keeps PER = np2 / NT <= 4 of the
// row's blocks in registers.
template <int D, int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                    int Lq, int nb, int np2, float scale, float tau, int k_min,
                                                    uint8_t* __restrict__ mask, int64_t pitch) {
  constexpr int PER = 4;
  constexpr int NWV = NT / 64;
  __shared__ float qv[D];
  __shared__ float fbuf[2][NWV];
  __shared__ int ibuf[2][NWV];
  __shared__ uint64_t kbuf[NWV];

  const int k = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int lane = t % 64, wave = t / 64;
  if (t < D) qv[t] = qp[((int64_t)h * Lq + k) * D + t];
  __syncthreads();

  // Keys of this thread's blocks j = t + r NT: ascending key = descending score, equal scores by ascending j;
  // positions past nb get the largest key and no weight.
  const float4* kh = reinterpret_cast<const float4*>(kp + (int64_t)h * nb * D);
  uint64_t key[PER];
  float w[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int j = t + r * NT;
    key[r] = ~0ull;
    if (j < nb) {
      float s = 0.f;
#pragma unroll 8
      for (int c = 0; c < D / 4; ++c) {
        const float4 kv = kh[(int64_t)j * (D / 4) + c];
        s += qv[4 * c] * kv.x + qv[4 * c + 1] * kv.y + qv[4 * c + 2] * kv.z + qv[4 * c + 3] * kv.w;
      }
      key[r] = ((uint64_t)(~ordered_bits(s * scale)) << 32) | (uint32_t)j;
    }
  }

  // Workgroup reductions in a fixed order (deterministic): butterfly within the wave, then the waves' totals
  // in wave order.  Two alternating LDS buffers let one barrier separate consecutive reductions.
  int parity = 0;
  auto sum_f = [&](float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) fbuf[parity][wave] = v;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int x = 0; x < NWV; ++x) tot += fbuf[parity][x];
    parity ^= 1;
    return tot;
  };
  auto sum_i = [&](int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) ibuf[parity][wave] = v;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int x = 0; x < NWV; ++x) tot += ibuf[parity][x];
    parity ^= 1;
    return tot;
  };

  // The smallest key is the row's maximum score.
  uint64_t kmin = key[0];
#pragma unroll
  for (int r = 1; r < PER; ++r) kmin = key[r] < kmin ? key[r] : kmin;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = shfl_xor64(kmin, off);
    kmin = o < kmin ? o : kmin;
  }
  if (lane == 0) kbuf[wave] = kmin;
  __syncthreads();
  kmin = kbuf[0];
  for (int x = 1; x < NWV; ++x) kmin = kbuf[x] < kmin ? kbuf[x] : kmin;
  const float smax = from_ordered_bits(~(uint32_t)(kmin >> 32));

  float part = 0.f;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    w[r] = key[r] != ~0ull ? expf(from_ordered_bits(~(uint32_t)(key[r] >> 32)) - smax) : 0.f;
    part += w[r];
  }
  const float target = tau * sum_f(part);

  // The smallest key threshold T whose blocks (key <= T) hold at least tau of the weight, found bit by bit
  // (bits 63..32: the score, bits 11..0: the block; no key has bits 31..12 set); n_tau = |{key <= T}|, at
  // least 1.
  auto mass_le = [&](uint64_t T) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < PER; ++r) m += key[r] <= T ? w[r] : 0.f;
    return sum_f(m);
  };
  auto count_le = [&](uint64_t T) {
    int c = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) c += key[r] <= T ? 1 : 0;
    return sum_i(c);
  };
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    if (bit == 31) bit = 11;
    const uint64_t probe = T | ((1ull << bit) - 1ull);
    if (!(mass_le(probe) >= target)) T |= 1ull << bit;
  }
  int cnt = count_le(T);
  const int n = min(nb, max(k_min, max(1, cnt)));
  if (n > cnt) {  // the Top-k floor (or the first block) asks for more: the n-th smallest key
    T = 0;
    for (int bit = 63; bit >= 0; --bit) {
      if (bit == 31) bit = 11;
      const uint64_t probe = T | ((1ull << bit) - 1ull);
      if (count_le(probe) < n) T |= 1ull << bit;
    }
  }

  uint8_t* row = mask + ((int64_t)h * Lq + k) * pitch;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int j = t + r * NT;
    if (j < pitch) row[j] = (j < nb && key[r] <= T) ? 1 : 0;
  }
  for (int i = np2 + t; i < pitch; i += NT) row[i] = 0;
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

hipError_t launch_pool(const Dims& g, const uint16_t* X, int n_blocks, const int32_t* block_ids, float* pooled,
                       hipStream_t stream) {
  if (n_blocks == 0) return hipSuccess;
  return g.d == 128 ? launch_pool_d<128>(g, X, n_blocks, block_ids, pooled, stream)
                    : launch_pool_d<64>(g, X, n_blocks, block_ids, pooled, stream);
}

hipError_t launch_select(const Dims& g, const float* q_pooled, const float* k_pooled, float scale, float tau,
                         int k_min, uint8_t* mask, int64_t pitch, hipStream_t stream) {
  if (g.Lq == 0) return hipSuccess;
  int np2 = 4;  // row length rounded up to a power of two
  while (np2 < g.nb) np2 <<= 1;
  const size_t lds = 0;
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
