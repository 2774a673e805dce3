// Block-mask materialisation from pooled tiles (SparSP paper, section 4.2: the block-sparse video DiT
// kernels it targets build their mask from pooled query and key tiles before attention starts; receivers
// combine remote key summaries with local query summaries and materialise the demand on the GPU).
//
// pool_kernel: mean of the real token rows of each block of b rows (one workgroup per (head, block);
// 16-byte loads, fp32 sums, row groups combined through LDS in a fixed order).  HBM-bound: it reads
// every token of K once.
//
// select_kernel: one workgroup per (head, R consecutive local query blocks); every thread keeps four or eight
// of each row's blocks in registers, and the R rows share every pooled-key read and every reduction.  Block
// scores s_j = scale <q, k_j> against every pooled key are keyed so that ascending key order is descending
// score (equal scores: ascending block); the softmax weights exp(s - max) are summed, and the smallest key
// threshold whose blocks hold at least tau of the weight is found bit by bit with workgroup reductions in
// a fixed order (no sort); a second, count-only search applies the Top-k floor k_min.  A row keeps the
// blocks at or below its threshold (a Top-p rule with a Top-k floor) and writes the uint8 mask row the
// demand union and the attention consume.  Integer counts and fixed-order fp32 sums make the result
// deterministic.
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

// Sum over the 64 lanes of a wave, the same in every lane, in a fixed order (deterministic): DPP steps within
// quads, half-rows and rows of 16, then the row broadcasts of lanes 15 and 31 gather the four rows into lane
// 63, which is read back.  Needs all 64 lanes active.
template <int Ctrl, int RowMask>
__device__ __forceinline__ int dpp_step(int v) {
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, RowMask, 0xF, false);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(dpp_step<0xB1, 0xF>(__float_as_int(v)));   // quad_perm [1, 0, 3, 2]
  v += __int_as_float(dpp_step<0x4E, 0xF>(__float_as_int(v)));   // quad_perm [2, 3, 0, 1]
  v += __int_as_float(dpp_step<0x141, 0xF>(__float_as_int(v)));  // row_half_mirror
  v += __int_as_float(dpp_step<0x140, 0xF>(__float_as_int(v)));  // row_mirror
  v += __int_as_float(dpp_step<0x142, 0xA>(__float_as_int(v)));  // row_bcast:15 into rows 1 and 3
  v += __int_as_float(dpp_step<0x143, 0xC>(__float_as_int(v)));  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_sum(int v) {
  v += dpp_step<0xB1, 0xF>(v);
  v += dpp_step<0x4E, 0xF>(v);
  v += dpp_step<0x141, 0xF>(v);
  v += dpp_step<0x140, 0xF>(v);
  v += dpp_step<0x142, 0xA>(v);
  v += dpp_step<0x143, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Monotone map of a float to an unsigned key (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// NT threads, each keeping PER >= np2 / NT blocks of each of the workgroup's R rows in registers: 256 threads,
// four blocks and four rows for rows of up to 1024 blocks; 512 threads, eight blocks and two rows up to 4096;
// 1024 threads, one row, eight or sixteen blocks up to 16384.  The
// R rows (consecutive local query blocks of one head) share every pooled-key read and every reduction.
template <int D, int NT, int R, int PER>
__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                    int Lq, int nb, int np2, float scale, float tau, int k_min,
                                                    uint8_t* __restrict__ mask, int64_t pitch) {
  constexpr int NWV = NT / 64;
  __shared__ float qv[R][D];
  __shared__ float fbuf[2][R][NWV];
  __shared__ int ibuf[2][R][NWV];
  __shared__ uint64_t kbuf[R][NWV];

  const int k0 = blockIdx.x * R, h = blockIdx.y, t = threadIdx.x;
  const int lane = t % 64, wave = t / 64;
  for (int i = t; i < R * D; i += NT) {
    const int rr = i / D, k = min(k0 + rr, Lq - 1);  // rows past Lq repeat the last one and are not written
    qv[rr][i % D] = qp[((int64_t)h * Lq + k) * D + i % D];
  }
  __syncthreads();

  // Keys of this thread's blocks j = t + r NT: ascending key = descending score, equal scores by ascending j;
  // positions past nb get the largest key and no weight.
  const float4* kh = reinterpret_cast<const float4*>(kp + (int64_t)h * nb * D);
  uint64_t key[R][PER];
  float w[R][PER];
  if constexpr (D == 64) {
    // d = 64: the dot products are split over quads of lanes: lane i of a quad holds elements [16 i, 16 i + 16)
    // of each row's pooled query in registers and computes that slice of the dot products of the blocks owned
    // by the quad's four threads (the quad reads each pooled-key row as one contiguous 256-byte span); the
    // slices are summed across the quad in a fixed order with DPP.  (At d = 128 the same split over eight
    // lanes measured slower than whole dot products per thread.)
    const int gi = lane % 4;
    float qs[R][16];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int e = 0; e < 16; ++e) qs[q][e] = qv[q][gi * 16 + e];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      float sc[R];
#pragma unroll
      for (int q = 0; q < R; ++q) sc[q] = 0.f;
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const int j = (t - gi + o) + r * NT;  // block of the quad's o-th thread (the same for the whole quad)
        float part[R];
#pragma unroll
        for (int q = 0; q < R; ++q) part[q] = 0.f;
        if (j < nb) {
          const float4* kr = kh + (int64_t)j * (D / 4) + gi * 4;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float4 kv = kr[c];
#pragma unroll
            for (int q = 0; q < R; ++q)
              part[q] += qs[q][4 * c] * kv.x + qs[q][4 * c + 1] * kv.y + qs[q][4 * c + 2] * kv.z + qs[q][4 * c + 3] * kv.w;
          }
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {
          float v = part[q];
          v += __int_as_float(dpp_step<0xB1, 0xF>(__float_as_int(v)));  // quad_perm [1, 0, 3, 2]
          v += __int_as_float(dpp_step<0x4E, 0xF>(__float_as_int(v)));  // quad_perm [2, 3, 0, 1]
          if (gi == o) sc[q] = v;
        }
      }
      const int j = t + r * NT;
#pragma unroll
      for (int q = 0; q < R; ++q)
        key[q][r] = j < nb ? ((uint64_t)(~ordered_bits(sc[q] * scale)) << 32) | (uint32_t)j : ~0ull;
    }
  } else {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int j = t + r * NT;
#pragma unroll
      for (int q = 0; q < R; ++q) key[q][r] = ~0ull;
      if (j < nb) {
        float s[R];
#pragma unroll
        for (int q = 0; q < R; ++q) s[q] = 0.f;
#pragma unroll 4
        for (int c = 0; c < D / 4; ++c) {
          const float4 kv = kh[(int64_t)j * (D / 4) + c];
#pragma unroll
          for (int q = 0; q < R; ++q)
            s[q] += qv[q][4 * c] * kv.x + qv[q][4 * c + 1] * kv.y + qv[q][4 * c + 2] * kv.z + qv[q][4 * c + 3] * kv.w;
        }
#pragma unroll
        for (int q = 0; q < R; ++q) key[q][r] = ((uint64_t)(~ordered_bits(s[q] * scale)) << 32) | (uint32_t)j;
      }
    }
  }

  // Workgroup reductions of R values at once, in a fixed order (deterministic): DPP within the wave, then the
  // waves' totals in wave order.  Two alternating LDS buffers let one barrier separate
  // consecutive reductions.
  int parity = 0;
  auto sum_f = [&](float (&v)[R]) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float ws = wave_sum(v[q]);
      if (lane == 0) fbuf[parity][q][wave] = ws;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < R; ++q) {
      float tot = 0.f;
#pragma unroll
      for (int x = 0; x < NWV; ++x) tot += fbuf[parity][q][x];
      v[q] = tot;
    }
    parity ^= 1;
  };
  auto sum_i = [&](int (&v)[R]) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int ws = wave_sum(v[q]);
      if (lane == 0) ibuf[parity][q][wave] = ws;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < R; ++q) {
      int tot = 0;
#pragma unroll
      for (int x = 0; x < NWV; ++x) tot += ibuf[parity][q][x];
      v[q] = tot;
    }
    parity ^= 1;
  };

  // The smallest key of a row is its maximum score.
  float target[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    uint64_t kmin = key[q][0];
#pragma unroll
    for (int r = 1; r < PER; ++r) kmin = key[q][r] < kmin ? key[q][r] : kmin;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t o = shfl_xor64(kmin, off);
      kmin = o < kmin ? o : kmin;
    }
    if (lane == 0) kbuf[q][wave] = kmin;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < R; ++q) {
    uint64_t kmin = kbuf[q][0];
    for (int x = 1; x < NWV; ++x) kmin = kbuf[q][x] < kmin ? kbuf[q][x] : kmin;
    const float smax = from_ordered_bits(~(uint32_t)(kmin >> 32));
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      w[q][r] = key[q][r] != ~0ull ? expf(from_ordered_bits(~(uint32_t)(key[q][r] >> 32)) - smax) : 0.f;
      part += w[q][r];
    }
    target[q] = part;
  }
  sum_f(target);
#pragma unroll
  for (int q = 0; q < R; ++q) target[q] *= tau;

  // Per row, the smallest key threshold T whose blocks (key <= T) hold at least tau of the weight, found bit by
  // bit (bits 63..32: the score, then the low bits a block index below np2 can have; no key has the bits in
  // between set); n_tau = |{key <= T}|, at least 1.
  const int jbits = 31 - __clz(np2);  // index bits a block of this row can have set
  uint64_t T[R];
#pragma unroll
  for (int q = 0; q < R; ++q) T[q] = 0;
  for (int bit = 63; bit >= 0; --bit) {
    if (bit == 31) bit = jbits - 1;
    float m[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const uint64_t probe = T[q] | ((1ull << bit) - 1ull);
      m[q] = 0.f;
#pragma unroll
      for (int r = 0; r < PER; ++r) m[q] += key[q][r] <= probe ? w[q][r] : 0.f;
    }
    sum_f(m);
#pragma unroll
    for (int q = 0; q < R; ++q)
      if (!(m[q] >= target[q])) T[q] |= 1ull << bit;
  }
  int cnt[R], n[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    cnt[q] = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) cnt[q] += key[q][r] <= T[q] ? 1 : 0;
  }
  sum_i(cnt);
  bool more = false;
#pragma unroll
  for (int q = 0; q < R; ++q) {
    n[q] = min(nb, max(k_min, max(1, cnt[q])));
    if (n[q] == nb && cnt[q] < nb) {  // every block: no search needed
      T[q] = ~0ull;
      cnt[q] = nb;
    }
    more |= n[q] > cnt[q];
  }
  if (more) {  // the Top-k floor (or the first block) asks for more: the n-th smallest key of those rows
    uint64_t T2[R];
#pragma unroll
    for (int q = 0; q < R; ++q) T2[q] = 0;
    for (int bit = 63; bit >= 0; --bit) {
      if (bit == 31) bit = jbits - 1;
      int c[R];
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const uint64_t probe = T2[q] | ((1ull << bit) - 1ull);
        c[q] = 0;
#pragma unroll
        for (int r = 0; r < PER; ++r) c[q] += key[q][r] <= probe ? 1 : 0;
      }
      sum_i(c);
#pragma unroll
      for (int q = 0; q < R; ++q)
        if (c[q] < n[q]) T2[q] |= 1ull << bit;
    }
#pragma unroll
    for (int q = 0; q < R; ++q)
      if (n[q] > cnt[q]) T[q] = T2[q];
  }

#pragma unroll
  for (int q = 0; q < R; ++q) {
    if (k0 + q >= Lq) break;
    uint8_t* row = mask + ((int64_t)h * Lq + k0 + q) * pitch;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int j = t + r * NT;
      if (j < pitch) row[j] = (j < nb && key[q][r] <= T[q]) ? 1 : 0;
    }
    for (int i = np2 + t; i < pitch; i += NT) row[i] = 0;
  }
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
  // Rows of up to 1024 blocks: 256 threads, four blocks per thread and four rows per workgroup; longer rows
  // (up to 4096 blocks): 512 threads, eight blocks per thread and two rows (1024 threads with one row, or two
  // and four rows of 1024 threads, measured slower); up to 8192 and 16384 blocks: 1024 threads, one row, eight
  // or sixteen blocks per thread.
  if (np2 <= 1024) {
    const dim3 grid((unsigned)((g.Lq + 3) / 4), (unsigned)g.H);
    if (g.d == 128)
      hipLaunchKernelGGL((select_kernel<128, 256, 4, 4>), grid, dim3(256), 0, stream, q_pooled, k_pooled, g.Lq, g.nb, np2,
                         scale, tau, k_min, mask, pitch);
    else
      hipLaunchKernelGGL((select_kernel<64, 256, 4, 4>), grid, dim3(256), 0, stream, q_pooled, k_pooled, g.Lq, g.nb, np2,
                         scale, tau, k_min, mask, pitch);
  } else if (np2 <= 4096) {
    const dim3 grid((unsigned)((g.Lq + 1) / 2), (unsigned)g.H);
    if (g.d == 128)
      hipLaunchKernelGGL((select_kernel<128, 512, 2, 8>), grid, dim3(512), 0, stream, q_pooled, k_pooled, g.Lq, g.nb,
                         np2, scale, tau, k_min, mask, pitch);
    else
      hipLaunchKernelGGL((select_kernel<64, 512, 2, 8>), grid, dim3(512), 0, stream, q_pooled, k_pooled, g.Lq, g.nb,
                         np2, scale, tau, k_min, mask, pitch);
  } else {
    const dim3 grid((unsigned)g.Lq, (unsigned)g.H);
    if (np2 <= 8192) {
      if (g.d == 128)
        hipLaunchKernelGGL((select_kernel<128, 1024, 1, 8>), grid, dim3(1024), 0, stream, q_pooled, k_pooled, g.Lq, g.nb,
                           np2, scale, tau, k_min, mask, pitch);
      else
        hipLaunchKernelGGL((select_kernel<64, 1024, 1, 8>), grid, dim3(1024), 0, stream, q_pooled, k_pooled, g.Lq, g.nb,
                           np2, scale, tau, k_min, mask, pitch);
    } else {
      if (g.d == 128)
        hipLaunchKernelGGL((select_kernel<128, 1024, 1, 16>), grid, dim3(1024), 0, stream, q_pooled, k_pooled, g.Lq,
                           g.nb, np2, scale, tau, k_min, mask, pitch);
      else
        hipLaunchKernelGGL((select_kernel<64, 1024, 1, 16>), grid, dim3(1024), 0, stream, q_pooled, k_pooled, g.Lq,
                           g.nb, np2, scale, tau, k_min, mask, pitch);
    }
  }
  return hipGetLastError();
}

}  // namespace sparsp
