// Block-sparse flash attention over the compacted K/V for one rank's local queries.
//
// SparSP paper (full text): section 2.2 gives O = softmax(Q K^T / sqrt(d)) V; Eq. 2 (section 4.1)
// restricts query block i to the key blocks j with M[h, i, j] = 1; section 2.3 describes consuming KV
// piece by piece with an online softmax.  One workgroup computes one (head, local query block) pair.
//
// Layout on gfx950.  Each wave owns 32 query rows and uses v_mfma_f32_32x32x16_bf16.  Scores are formed
// transposed, S^T = K Q^T (M = keys, N = query rows, K = d), so that in the accumulator every lane holds
// a single query row (lane % 32) and 16 keys of each 32-key group; the two lane halves split the keys.
// The softmax statistics are therefore per-lane scalars, and the only cross-lane step per stage is one
// exchange between lanes l and l ^ 32.  The exponentiated scores already sit where the B operand of the
// second product wants them: O^T += V^T P^T (M = d, N = query rows, K = keys) takes P^T straight from the
// score registers (converted to bf16), and V^T comes from the transposed V half of the packed slot.
//
// Pipeline.  Every selected key block is consumed in stages of 64 keys.  A stage (64 K rows and the
// matching 64 columns of V^T) is staged in LDS; the next stage's global loads are issued into registers
// before the current stage is computed, so the load latency hides behind the MFMA work, and two
// workgroups share a CU.  LDS rows are XOR-swizzled in 16-byte chunks so that both the 16-byte stores and
// the MFMA fragment reads are free of bank conflicts without padding.
//
// Softmax.  The running maximum is only raised when some row of the wave grows by more than 2^8 (a
// wave-uniform decision); until then probabilities are taken against the stale maximum, which is exact in
// real arithmetic because numerator and denominator share it, and saves the O rescale on most stages.
#include <math.h>

#include "sparsp_internal.h"

namespace sparsp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;  // 16 bytes; a native vector so it stays in VGPRs
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kStageKeys = 64;     // keys per pipeline stage
constexpr int kListCap = 512;      // selected blocks listed per pass over the mask row
constexpr float kRescaleLog2 = 8.f;

template <int D, int B>
struct Tile {
  static constexpr int NW = B / 32;                      // waves, 32 query rows each
  static constexpr int NT = NW * 64;                     // threads
  static constexpr int NST = B / kStageKeys;             // stages per key block
  // LDS row pitches.  The LDS serves 128 bytes per clock from 32 four-byte banks: 8 lanes of a 16-byte
  // access or 16 lanes of an 8-byte access.  The fragment reads take one column of consecutive rows, so a
  // K row pitch of 4 (mod 32) words and a V^T row pitch of 2 (mod 32) words put those lanes on distinct
  // banks; the stores write 128 contiguous bytes per clock.
  static constexpr int KP = D * 2 + 16;                  // bytes per K row, 16-byte aligned
  static constexpr int VP = kStageKeys * 2 + 8;          // bytes per V^T row, 8-byte aligned
  static constexpr int KBYTES = kStageKeys * KP;         // K part of a stage buffer
  static constexpr int STAGE = KBYTES + D * VP;          // one stage buffer
  static constexpr int KCH = kStageKeys * D / 8;         // 16-byte chunks of K per stage (same for V^T)
  static constexpr int KCPT = KCH / NT;                  // K chunks per thread per stage (same for V^T)
  static constexpr int NDT = D / 32;                     // 32-row tiles of O^T
  static constexpr int NQF = D / 16;                     // Q fragments along d
  static constexpr int64_t SLOT = 2ll * B * D;           // elements per packed slot
  static_assert(KCH % NT == 0, "stage must split evenly over the threads");
};

// Issue this thread's global loads of stage hh of a packed slot (K rows hh*64.., V^T columns hh*64..).
template <int D, int B, int N2>
__device__ __forceinline__ void load_stage(u32x4 (&pre)[N2], const char* __restrict__ slot, int hh, int t) {
  using T = Tile<D, B>;
  static_assert(N2 == 2 * T::KCPT, "one register per chunk");
  const char* k = slot + hh * (kStageKeys * D * 2);
  const char* v = slot + (int64_t)B * D * 2 + hh * (kStageKeys * 2);
#pragma unroll
  for (int i = 0; i < T::KCPT; ++i) {
    const int q = t + i * T::NT;
    pre[i] = *reinterpret_cast<const u32x4*>(k + (unsigned)((q / (D / 8)) * D + (q % (D / 8)) * 8) * 2u);
    pre[T::KCPT + i] = *reinterpret_cast<const u32x4*>(v + (unsigned)((q / 8) * B + (q % 8) * 8) * 2u);
  }
}

// Write the registers of the loaded stage into an LDS stage buffer.
template <int D, int B, int N2>
__device__ __forceinline__ void store_stage(const u32x4 (&pre)[N2], unsigned char* buf, int t) {
  using T = Tile<D, B>;
#pragma unroll
  for (int i = 0; i < T::KCPT; ++i) {
    const int q = t + i * T::NT;
    *reinterpret_cast<u32x4*>(buf + (q / (D / 8)) * T::KP + (q % (D / 8)) * 16) = pre[i];
    unsigned char* vrow = buf + T::KBYTES + (q / 8) * T::VP + (q % 8) * 16;
    *reinterpret_cast<u32x2*>(vrow) = pre[T::KCPT + i].xy;
    *reinterpret_cast<u32x2*>(vrow + 8) = pre[T::KCPT + i].zw;
  }
}

template <int D, int B>
__global__ __launch_bounds__(2 * B) __attribute__((amdgpu_waves_per_eu(2, 2))) void bsa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ mask, int64_t pitch,
    const int32_t* __restrict__ slot_of, const uint16_t* __restrict__ packed, int slot_capacity, float scale_log2,
    int Lq, int nb, int N, float* __restrict__ O, float* __restrict__ lse) {
  using T = Tile<D, B>;
  __shared__ __align__(16) unsigned char sStage[2][T::STAGE];
  __shared__ int sList[kListCap];
  __shared__ int sWaveCnt[T::NW];

  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wid / Lq, k = wid - h * Lq;
  const int t = threadIdx.x, lane = t % 64, wave = t / 64;
  const int qr = lane % 32, half = lane / 32;

  // Q^T fragments (B operand of S^T = K Q^T): row qr of this wave, d = 16f + 8*half .. +7.
  const int64_t row = (int64_t)h * Lq * B + (int64_t)k * B + wave * 32 + qr;
  bf16x8 qf[T::NQF];
#pragma unroll
  for (int f = 0; f < T::NQF; ++f) qf[f] = *reinterpret_cast<const bf16x8*>(Q + row * D + f * 16 + half * 8);

  f32x16 oacc[T::NDT];
#pragma unroll
  for (int i = 0; i < T::NDT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
  float m_run = -INFINITY;  // maximum the probabilities are taken against (log2-scaled logits)
  float l_run = 0.f;        // sum of exp2(x - m_run) over this lane's keys

  const uint8_t* mrow = mask + ((int64_t)h * Lq + k) * pitch;
  const int32_t* sof = slot_of + (int64_t)h * nb;
  const int tail_valid = N - (nb - 1) * B;  // real keys in the last block, 1..B
  const char* pk = reinterpret_cast<const char*>(packed);

  int col = 0;
  while (col < nb) {
    // List the selected blocks of the next columns (ascending j) as (slot << 1 | is_last_block).
    int total = 0;
    while (col < nb && total <= kListCap - T::NT) {
      const int j = col + t;
      int slot = -1;
      if (j < nb && mrow[j] != 0) {
        slot = sof[j];
        if (slot >= slot_capacity) slot = -1;
      }
      const uint64_t bal = __ballot(slot >= 0);
      if (lane == 0) sWaveCnt[wave] = __popcll(bal);
      __syncthreads();
      int off = total, add = 0;
#pragma unroll
      for (int w = 0; w < T::NW; ++w) {
        const int c = sWaveCnt[w];
        off += w < wave ? c : 0;
        add += c;
      }
      if (slot >= 0) sList[off + __popcll(bal & ((1ull << lane) - 1ull))] = (slot << 1) | (j == nb - 1 ? 1 : 0);
      total += add;
      col += T::NT;
      __syncthreads();
    }

    const int nstage = total * T::NST;
    u32x4 pre[2 * T::KCPT];
    if (nstage > 0) {
      const int c0 = __builtin_amdgcn_readfirstlane(sList[0]);
      load_stage<D, B>(pre, pk + (int64_t)(c0 >> 1) * (T::SLOT * 2), 0, t);
    }

    for (int st = 0; st < nstage; ++st) {
      // Double-buffered stages: buffer st&1 was last read by stage st-2, which every wave finished
      // before the barrier of stage st-1.
      unsigned char* buf = sStage[st & 1];
      store_stage<D, B>(pre, buf, t);
      const int code = __builtin_amdgcn_readfirstlane(sList[st / T::NST]);
      const int hh = st % T::NST;
      if (st + 1 < nstage) {
        const int cn = __builtin_amdgcn_readfirstlane(sList[(st + 1) / T::NST]);
        load_stage<D, B>(pre, pk + (int64_t)(cn >> 1) * (T::SLOT * 2), (st + 1) % T::NST, t);
      }
      __syncthreads();

      // S^T = K Q^T for the two 32-key groups of the stage (raw scores).
      const unsigned char* kb = buf + qr * T::KP + half * 16;
      f32x16 sacc[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        sacc[g] = mfma32(*reinterpret_cast<const bf16x8*>(kb + g * 32 * T::KP), qf[0], f32x16{});
#pragma unroll
        for (int f = 1; f < T::NQF; ++f)
          sacc[g] = mfma32(*reinterpret_cast<const bf16x8*>(kb + g * 32 * T::KP + f * 32), qf[f], sacc[g]);
      }

      // sacc[g][4i + r] is key 64*hh + 32g + 8i + 4*half + r of query row qr.  Key tokens past N (only in
      // the last block) are masked; the branch is uniform.
      if ((code & 1) && hh * kStageKeys + kStageKeys > tail_valid) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int key = hh * kStageKeys + g * 32 + (x / 4) * 8 + half * 4 + (x % 4);
            if (key >= tail_valid) sacc[g][x] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[g][x]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;  // scale_log2 > 0: the max commutes with scaling
      if (__ballot(mx > m_run + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < T::NDT; ++i) oacc[i] *= alpha;
      }

      bf16x8 pf[2][2];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[g][x], scale_log2, -m_run));
          l_run += p;
          pf[g][x / 8][x % 8] = (__bf16)p;
        }

      // O^T += V^T P^T.  MFMA (g, hf) covers keys 32g + 16hf + {0..3, 8..11} + 4*half of the stage.
      const unsigned char* vb = buf + T::KBYTES + qr * T::VP + half * 8;
#pragma unroll
      for (int i = 0; i < T::NDT; ++i)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const unsigned char* v = vb + i * 32 * T::VP + (g * 32 + hf * 16) * 2;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(v);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(v + 16);
            oacc[i] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf[g][hf], oacc[i]);
          }
    }
    __syncthreads();  // sList and the stage buffers are reused by the next pass
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* orow = O + row * D;
#pragma unroll
  for (int i = 0; i < T::NDT; ++i)
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
