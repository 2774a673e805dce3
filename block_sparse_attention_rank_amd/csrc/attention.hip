// Block-sparse flash attention over the compacted K/V for one rank's local queries.
//
// SparSP paper (full text): section 2.2 gives O = softmax(Q K^T / sqrt(d)) V; Eq. 2 (section 4.1)
// restricts query block i to the key blocks j with M[h, i, j] = 1; section 2.3 describes consuming KV
// piece by piece with an online softmax.  One workgroup computes one (head, local query block) pair.
//
// Layout on gfx950.  Each wave owns 32 query rows and uses v_mfma_f32_32x32x16_bf16.  Scores are formed
// transposed, S^T = K Q^T (M = keys, N = query rows, K = d), so that in the accumulator every lane holds
// a single query row (lane % 32) and 16 keys of each 32-key group; the two lane halves split the keys.
// The softmax statistics are therefore per-lane scalars, and the only cross-lane step per tile is one
// exchange between lanes l and l ^ 32.  The exponentiated scores already sit where the B operand of the
// second product wants them: O^T += V^T P^T (M = d, N = query rows, K = keys) takes P^T straight from the
// score registers (converted to bf16), and V^T comes from the transposed V half of the packed slot.
// K and V^T tiles are staged in LDS with a 16-byte row pad so the fragment reads are bank-conflict-free.
#include <math.h>

#include "sparsp_internal.h"

namespace sparsp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int B>
__global__ __launch_bounds__(2 * B) void bsa_fwd_kernel(const uint16_t* __restrict__ Q,
                                                        const uint8_t* __restrict__ mask, int64_t pitch,
                                                        const int32_t* __restrict__ slot_of,
                                                        const uint16_t* __restrict__ packed, int slot_capacity,
                                                        float scale_log2, int Lq, int nb, int N,
                                                        float* __restrict__ O, float* __restrict__ lse) {
  constexpr int NW = B / 32;   // waves; each owns 32 query rows
  constexpr int NT = NW * 64;  // threads
  constexpr int KP = D + 8;    // K tile row pitch (elements)
  constexpr int VP = B + 8;    // V^T tile row pitch (elements)
  constexpr int NKG = B / 32;  // 32-key groups per tile
  constexpr int NDT = D / 32;  // 32-row tiles of O^T
  constexpr int NQF = D / 16;  // Q fragments along d
  constexpr int64_t kSlotElems = 2ll * B * D;

  __shared__ __align__(16) uint16_t sK[B * KP];
  __shared__ __align__(16) uint16_t sV[D * VP];
  __shared__ int sList[NT];
  __shared__ int sWaveCnt[NW];

  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wid / Lq, k = wid - h * Lq;
  const int t = threadIdx.x, lane = t % 64, wave = t / 64;
  const int qr = lane % 32, half = lane / 32;

  // Q^T fragments (B operand of S^T = K Q^T): row qr of this wave, d = 16f + 8*half .. +7.
  const int64_t row = (int64_t)h * Lq * B + (int64_t)k * B + wave * 32 + qr;
  bf16x8 qf[NQF];
#pragma unroll
  for (int f = 0; f < NQF; ++f) qf[f] = *reinterpret_cast<const bf16x8*>(Q + row * D + f * 16 + half * 8);

  f32x16 oacc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY;  // running max of the log2-scaled logits of this row
  float l_run = 0.f;        // running sum of exp2(x - m_run) over this lane's keys

  const uint8_t* mrow = mask + ((int64_t)h * Lq + k) * pitch;
  const int32_t* sof = slot_of + (int64_t)h * nb;
  const int tail_valid = N - (nb - 1) * B;  // real keys in the last block, 1..B

  for (int c0 = 0; c0 < nb; c0 += NT) {
    // The selected blocks of this chunk of the mask row, in ascending j, as (slot << 1 | is_last_block).
    const int j = c0 + t;
    int slot = -1;
    if (j < nb && mrow[j] != 0) {
      slot = sof[j];
      if (slot >= slot_capacity) slot = -1;
    }
    const uint64_t bal = __ballot(slot >= 0);
    if (lane == 0) sWaveCnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = sWaveCnt[w];
      off += w < wave ? c : 0;
      total += c;
    }
    if (slot >= 0) sList[off + __popcll(bal & ((1ull << lane) - 1ull))] = (slot << 1) | (j == nb - 1 ? 1 : 0);
    __syncthreads();

    for (int e = 0; e < total; ++e) {
      const int code = sList[e];
      const bool last = code & 1;
      const uint16_t* src = packed + (int64_t)(code >> 1) * kSlotElems;
#pragma unroll
      for (int c = t; c < B * D / 8; c += NT) {
        const int rr = c / (D / 8), cc = (c % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(sK + rr * KP + cc) = *reinterpret_cast<const uint4*>(src + c * 8);
      }
#pragma unroll
      for (int c = t; c < D * B / 8; c += NT) {
        const int rr = c / (B / 8), cc = (c % (B / 8)) * 8;
        *reinterpret_cast<uint4*>(sV + rr * VP + cc) = *reinterpret_cast<const uint4*>(src + B * D + c * 8);
      }
      __syncthreads();

      // S^T = K Q^T for the 32-key groups of the tile.
      f32x16 sacc[NKG];
#pragma unroll
      for (int g = 0; g < NKG; ++g) {
#pragma unroll
        for (int x = 0; x < 16; ++x) sacc[g][x] = 0.f;
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (g * 32 + qr) * KP + f * 16 + half * 8);
          sacc[g] = mfma32(a, qf[f], sacc[g]);
        }
      }

      // Online softmax.  sacc[g][4i + r] is key 32g + 8i + 4*half + r of query row qr.
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < NKG; ++g)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          float v = sacc[g][x] * scale_log2;
          if (last) {
            const int key = g * 32 + (x / 4) * 8 + half * 4 + (x % 4);
            if (key >= tail_valid) v = -INFINITY;
          }
          sacc[g][x] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;

      bf16x8 pf[NKG][2];
      float lsum = 0.f;
#pragma unroll
      for (int g = 0; g < NKG; ++g)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float p = __builtin_amdgcn_exp2f(sacc[g][x] - m_new);
          lsum += p;
          pf[g][x / 8][x % 8] = (__bf16)p;
        }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int i = 0; i < NDT; ++i) oacc[i] *= alpha;

      // O^T += V^T P^T.  MFMA (g, hf) covers keys 32g + 16hf + {0..3, 8..11} + 4*half for this lane.
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int g = 0; g < NKG; ++g)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const uint16_t* vr = sV + (i * 32 + qr) * VP + g * 32 + hf * 16 + half * 4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 8);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[i] = mfma32(a, pf[g][hf], oacc[i]);
          }
      __syncthreads();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* orow = O + row * D;
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = make_float4(oacc[i][4 * q + 0] * inv, oacc[i][4 * q + 1] * inv, oacc[i][4 * q + 2] * inv,
                                   oacc[i][4 * q + 3] * inv);
      *reinterpret_cast<float4*>(orow + i * 32 + q * 8 + half * 4) = v;
    }
  if (half == 0) lse[row] = l_tot > 0.f ? m_run * 0.69314718055994531f + logf(l_tot) : -INFINITY;
}

template <int D, int B>
hipError_t launch_attention_t(const Dims& g, const uint16_t* Q, const uint8_t* mask, int64_t pitch,
                              const int32_t* slot_of, const uint16_t* packed, int32_t slot_capacity,
                              float softmax_scale, float* O, float* lse, hipStream_t stream) {
  const int64_t items = (int64_t)g.H * g.Lq;
  if (items == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL((bsa_fwd_kernel<D, B>), dim3((unsigned)items), dim3(2 * B), 0, stream, Q, mask, pitch,
                     slot_of, packed, slot_capacity, scale_log2, g.Lq, g.nb, g.N, O, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Dims& g, const uint16_t* Q, const uint8_t* mask, int64_t pitch,
                            const int32_t* slot_of, const uint16_t* packed, int32_t slot_capacity,
                            float softmax_scale, float* O, float* lse, hipStream_t stream) {
  if (g.d == 128 && g.b == 128)
    return launch_attention_t<128, 128>(g, Q, mask, pitch, slot_of, packed, slot_capacity, softmax_scale, O, lse,
                                        stream);
  if (g.d == 64 && g.b == 64)
    return launch_attention_t<64, 64>(g, Q, mask, pitch, slot_of, packed, slot_capacity, softmax_scale, O, lse,
                                      stream);
  if (g.d == 128 && g.b == 64)
    return launch_attention_t<128, 64>(g, Q, mask, pitch, slot_of, packed, slot_capacity, softmax_scale, O, lse,
                                       stream);
  return launch_attention_t<64, 128>(g, Q, mask, pitch, slot_of, packed, slot_capacity, softmax_scale, O, lse,
                                     stream);
}

}  // namespace sparsp
