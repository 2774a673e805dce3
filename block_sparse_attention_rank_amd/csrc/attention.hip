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

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kStageKeys = 64;     // keys per pipeline stage
constexpr int kListCap = 1024;     // selected blocks listed per pass over the mask row
constexpr float kRescaleLog2 = 8.f;

template <int D, int B>
struct Tile {
  static constexpr int NW = B / 32;                      // waves, 32 query rows each
  static constexpr int NT = NW * 64;                     // threads
  static constexpr int NST = B / kStageKeys;             // stages per key block
  static constexpr int KP = D * 2 + 16;                  // LDS bytes per K row (16-byte pad)
  static constexpr int VP = kStageKeys * 2 + 16;         // LDS bytes per V^T row (16-byte pad)
  static constexpr int KBYTES = kStageKeys * KP;         // K part of a stage in LDS
  static constexpr int VBYTES = D * VP;                  // V^T part of a stage in LDS
  static constexpr int KCH = kStageKeys * D / 8;         // 16-byte chunks of K per stage
  static constexpr int CH = 2 * KCH;                     // ... of K and V^T
  static constexpr int CPT = CH / NT;                    // chunks per thread per stage
  static constexpr int NDT = D / 32;                     // 32-row tiles of O^T
  static constexpr int NQF = D / 16;                     // Q fragments along d
  static constexpr int64_t SLOT = 2ll * B * D;           // elements per packed slot
  static_assert(CH % NT == 0, "stage must split evenly over the threads");
};

// Global element offset (within a slot) and LDS byte offset of the q-th 16-byte chunk of stage hh.
// Rows are padded by 16 bytes: consecutive rows start 4 banks apart, so the 8 (16-byte reads) or 16
// (8-byte reads) lanes the LDS serves per cycle, which read one column of consecutive rows, never collide,
// and every fragment address is a per-lane base plus a compile-time offset.
template <int D, int B>
__device__ __forceinline__ void stage_chunk(int q, int hh, int64_t& gofs, int& lofs) {
  using T = Tile<D, B>;
  if (q < T::KCH) {
    const int r = q / (D / 8), c = q % (D / 8);
    gofs = (int64_t)(hh * kStageKeys + r) * D + c * 8;
    lofs = r * T::KP + c * 16;
  } else {
    const int qq = q - T::KCH;
    const int dd = qq / 8, c = qq % 8;
    gofs = (int64_t)B * D + (int64_t)dd * B + hh * kStageKeys + c * 8;
    lofs = T::KBYTES + dd * T::VP + c * 16;
  }
}

// Issue the global loads of stage hh of packed slot `slot` into this thread's registers.
template <int D, int B, int NPRE>
__device__ __forceinline__ void load_stage(u32x4 (&pre)[NPRE], const uint16_t* __restrict__ packed, int slot,
                                           int hh, int t) {
  using T = Tile<D, B>;
  static_assert(NPRE == T::CPT, "one register per chunk");
  const uint16_t* src = packed + (int64_t)slot * T::SLOT;
#pragma unroll
  for (int i = 0; i < T::CPT; ++i) {
    int64_t g;
    int l;
    stage_chunk<D, B>(t + i * T::NT, hh, g, l);
    pre[i] = *reinterpret_cast<const u32x4*>(src + g);
  }
}

template <int D, int B>
__global__ __launch_bounds__(2 * B) __attribute__((amdgpu_waves_per_eu(2, 2))) void bsa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ mask, int64_t pitch,
    const int32_t* __restrict__ slot_of, const uint16_t* __restrict__ packed, int slot_capacity, float scale_log2,
    int Lq, int nb, int N, float* __restrict__ O, float* __restrict__ lse) {
  using T = Tile<D, B>;
  __shared__ __align__(16) unsigned char sStage[T::KBYTES + T::VBYTES];
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

  // LDS bases of this lane's fragment reads: K row qr (+32 per key group), V^T row qr (+32 per d tile).
  const unsigned char* kbase = sStage + qr * T::KP + half * 16;
  const unsigned char* vbase = sStage + T::KBYTES + qr * T::VP + half * 8;

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
    u32x4 pre[T::CPT];
    if (nstage > 0) load_stage<D, B>(pre, packed, sList[0] >> 1, 0, t);

    for (int st = 0; st < nstage; ++st) {
      const int code = sList[st / T::NST];
      const int hh = st % T::NST;
      const bool last = (code & 1) != 0;
      __syncthreads();  // every wave is done reading the previous stage
#pragma unroll
      for (int i = 0; i < T::CPT; ++i) {
        int64_t g;
        int l;
        stage_chunk<D, B>(t + i * T::NT, hh, g, l);
        *reinterpret_cast<u32x4*>(sStage + l) = pre[i];
      }
      if (st + 1 < nstage) load_stage<D, B>(pre, packed, sList[(st + 1) / T::NST] >> 1, (st + 1) % T::NST, t);
      __syncthreads();

      // S^T = K Q^T for the two 32-key groups of the stage.
      f32x16 sacc[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int x = 0; x < 16; ++x) sacc[g][x] = 0.f;
#pragma unroll
        for (int f = 0; f < T::NQF; ++f)
          sacc[g] = mfma32(*reinterpret_cast<const bf16x8*>(kbase + g * 32 * T::KP + f * 32), qf[f], sacc[g]);
      }

      // sacc[g][4i + r] is key 64*hh + 32g + 8i + 4*half + r of query row qr.
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          float v = sacc[g][x] * scale_log2;
          if (last) {
            const int key = hh * kStageKeys + g * 32 + (x / 4) * 8 + half * 4 + (x % 4);
            if (key >= tail_valid) v = -INFINITY;
          }
          sacc[g][x] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
          const float p = __builtin_amdgcn_exp2f(sacc[g][x] - m_run);
          l_run += p;
          pf[g][x / 8][x % 8] = (__bf16)p;
        }

      // O^T += V^T P^T.  MFMA (g, hf) covers keys 32g + 16hf + {0..3, 8..11} + 4*half of the stage.
#pragma unroll
      for (int i = 0; i < T::NDT; ++i)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const unsigned char* vb = vbase + i * 32 * T::VP + (g * 32 + hf * 16) * 2;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vb);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vb + 16);
            oacc[i] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf[g][hf], oacc[i]);
          }
    }
    __syncthreads();  // sList is rebuilt by the next pass
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
