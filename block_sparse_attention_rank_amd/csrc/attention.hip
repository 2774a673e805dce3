// Block-sparse flash attention over the compacted K/V for one rank's local queries.
//
// SparSP paper (full text): section 2.2 gives O = softmax(Q K^T / sqrt(d)) V; Eq. 2 (section 4.1)
// restricts query block i to the key blocks j with M[h, i, j] = 1; section 2.3 describes consuming KV
// piece by piece with an online softmax.  One workgroup computes one (head, local query block) pair.
//
// Layout on gfx950.  Each wave owns 32 query rows and uses v_mfma_f32_32x32x16_bf16.  Scores are formed
// transposed, S^T = K Q^T (M = keys, N = query rows, K = d), so that in the accumulator every lane holds
// a single query row (lane % 32) and 16 keys of each 32-key group; the two lane halves split the keys.
// The softmax statistics are per-lane scalars.  The exponentiated scores already sit where the B operand
// of the second product wants them: O^T += V^T P^T (M = d, N = query rows, K = keys) takes P^T straight
// from the score registers (converted to bf16), and V^T comes from the transposed V half of the packed
// slot.  The K rows of a stage are fed to the first product in a permuted order (bits 2 and 3 of the row
// index swapped) so that each lane's eight probabilities of a 16-key MFMA step are eight consecutive
// keys: every V^T fragment is then one 16-byte LDS read.
//
// Pipeline.  Every selected key block is consumed in stages of 64 keys.  A stage (64 K rows and the
// matching 64 columns of V^T, 2 x 64 x d bf16) is copied from global memory straight into LDS with
// global_load_lds_dwordx4 (no register staging); the next stage's copy is issued before the current one
// is computed, into the other of two LDS buffers, and two workgroups share a CU.  LDS rows are
// XOR-swizzled in 16-byte chunks (chunk c of row m sits at c ^ (m & 7)), which keeps the MFMA fragment
// reads free of bank conflicts; each lane's fragment addresses are fixed per kernel and the buffer, key
// group and d tile are immediate offsets.
//
// Softmax.  The running maximum is only raised when some row of the wave grows by more than 2^8 (a
// wave-uniform decision); until then probabilities are taken against the stale maximum, which is exact in
// real arithmetic because numerator and denominator share it.  The common path therefore needs no
// cross-lane step: the two halves of a row exchange their maxima (v_permlane32_swap) only when the
// maximum moves, and their partial sums once at the end.
#include <math.h>

#include "sparsp_internal.h"

namespace sparsp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max over lanes l and l ^ 32 (the two halves of a query row), without LDS.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): this lane's LDS-direct copies are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

constexpr int kStageKeys = 64;     // keys per pipeline stage
constexpr int kListCap = 512;      // selected blocks listed per pass over the mask row
constexpr float kRescaleLog2 = 8.f;

template <int D, int B>
struct Tile {
  static constexpr int NW = B / 32;                      // waves, 32 query rows each
  static constexpr int NT = NW * 64;                     // threads
  static constexpr int NST = B / kStageKeys;             // stages per key block
  static constexpr int KROW = D * 2;                     // bytes per K row of a stage
  static constexpr int KBYTES = kStageKeys * KROW;       // K part of a stage buffer
  static constexpr int VROW = kStageKeys * 2;            // bytes per V^T row of a stage (128)
  static constexpr int STAGE = KBYTES + D * VROW;        // one stage buffer
  static constexpr int CH = kStageKeys * D / 8;          // 16-byte chunks of K (and of V^T) per stage
  static constexpr int CPT = CH / NT;                    // K (and V^T) chunks per thread per stage
  static constexpr int NDT = D / 32;                     // 32-row tiles of O^T
  static constexpr int NQF = D / 16;                     // Q fragments along d
  static constexpr int64_t SLOT_BYTES = 4ll * B * D;     // bytes per packed slot
  static_assert(CH % NT == 0, "stage must split evenly over the threads");
  static_assert(NT * 16 == 64 * 16 * NW, "one 1 KiB LDS span per wave and copy");
  static_assert(2 * STAGE <= 65536, "LDS offsets must fit the 16-bit immediate");
};

// Stage-invariant parts of this lane's copies.  Copy i of wave w fills LDS chunks (i*NW + w)*64 + lane,
// 16 bytes per lane, of the K part and of the V^T part.
template <int D, int B>
struct CopyPlan {
  using T = Tile<D, B>;
  uint32_t koff[T::CPT];  // byte offset inside the slot's K part (stage 0)
  uint32_t voff[T::CPT];  // byte offset inside the slot (V^T part, stage 0)

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int q = (i * T::NW + wave) * 64 + lane;
      // K: LDS row m, chunk position cp holds logical chunk cp ^ (m & 7) of key sigma(m).
      const int m = q / (D / 8), cp = q % (D / 8);
      const int c = cp ^ (m & 7);
      const int key = (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
      koff[i] = (uint32_t)(key * (D * 2) + c * 16);
      // V^T: LDS row e (a d index), chunk position cp holds keys 8 * (cp ^ (e & 7)) .. +7.
      const int e = q / 8, vp = q % 8;
      const int vc = vp ^ (e & 7);
      voff[i] = (uint32_t)(B * D * 2 + e * (B * 2) + vc * 16);
    }
  }

  // Copy stage hh of the slot at `slot` into the LDS stage buffer `buf`.
  __device__ __forceinline__ void issue(const char* slot, int hh, unsigned char* buf, int wave) const {
    const char* k = slot + hh * T::KBYTES;
    const char* v = slot + hh * T::VROW;
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      __builtin_amdgcn_global_load_lds(k + koff[i], (lds_void*)(buf + (i * T::NW + wave) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(v + voff[i], (lds_void*)(buf + T::KBYTES + (i * T::NW + wave) * 1024), 16,
                                       0, 0);
    }
  }
};

// One stage: scores for 64 keys, online-softmax update, O^T += V^T P^T.
template <int D, int B>
__device__ __forceinline__ void stage_compute(const unsigned char* buf, const uint32_t (&kread)[Tile<D, B>::NQF],
                                              const uint32_t (&vread)[4], const bf16x8 (&qf)[Tile<D, B>::NQF],
                                              f32x16 (&oacc)[Tile<D, B>::NDT], float& m_run, float& l_run,
                                              float scale_log2, int lim) {
  using T = Tile<D, B>;
  // S^T = K Q^T for the two 32-key groups of the stage (raw scores).
  f32x16 sacc[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    sacc[g] = f32x16{};
#pragma unroll
    for (int f = 0; f < T::NQF; ++f)
      sacc[g] = mfma32(*reinterpret_cast<const bf16x8*>(buf + kread[f] + g * 32 * T::KROW), qf[f], sacc[g]);
  }

  // sacc[g][4i + r] is key 32g + 16(i >> 1) + 8 half + 4(i & 1) + r of the stage for query row lane % 32.
  // Keys at or past `lim` (relative to 8 half) are padding of the last block; the branch is uniform.
  if (lim < kStageKeys) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int c = 32 * g + 16 * (x / 8) + 4 * ((x / 4) % 2) + (x % 4);
        if (c >= lim) sacc[g][x] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[g][x]);
  mx *= scale_log2;  // scale_log2 > 0: the max commutes with scaling
  if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {
    const float m_new = fmaxf(m_run, max_halves(mx));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < T::NDT; ++i) oacc[i] *= alpha;
  }

  bf16x8 pf[4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[g][x], scale_log2, -m_run));
      l_run += p;
      pf[2 * g + x / 8][x % 8] = (__bf16)p;
    }

  // O^T += V^T P^T: step a covers keys 16a + 8 half + 0..7 of the stage, which is one V^T fragment.
#pragma unroll
  for (int i = 0; i < T::NDT; ++i)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      oacc[i] = mfma32(*reinterpret_cast<const bf16x8*>(buf + T::KBYTES + vread[a] + i * 32 * T::VROW), pf[a],
                       oacc[i]);
}

template <int D, int B>
__global__ __launch_bounds__(2 * B) __attribute__((amdgpu_waves_per_eu(2, 2))) void bsa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ mask, int64_t pitch,
    const int32_t* __restrict__ slot_of, const uint16_t* __restrict__ packed, int slot_capacity, float scale_log2,
    int Lq, int nb, int N, float* __restrict__ O, float* __restrict__ lse) {
  using T = Tile<D, B>;
  __shared__ __align__(1024) unsigned char sStage0[T::STAGE];
  __shared__ __align__(1024) unsigned char sStage1[T::STAGE];
  __shared__ int sList[kListCap];
  __shared__ int sWaveCnt[T::NW];

  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wid / Lq, k = wid - h * Lq;
  const int t = threadIdx.x, lane = t % 64;
  const int wave = __builtin_amdgcn_readfirstlane(t / 64);
  const int qr = lane % 32, half = lane / 32;

  // Q^T fragments (B operand of S^T = K Q^T): row qr of this wave, d = 16f + 8*half .. +7.
  const int64_t row = (int64_t)h * Lq * B + (int64_t)k * B + wave * 32 + qr;
  bf16x8 qf[T::NQF];
#pragma unroll
  for (int f = 0; f < T::NQF; ++f) qf[f] = *reinterpret_cast<const bf16x8*>(Q + row * D + f * 16 + half * 8);

  // This lane's LDS fragment addresses inside a stage buffer (swizzle key qr & 7 for every row it reads).
  uint32_t kread[T::NQF], vread[4];
#pragma unroll
  for (int f = 0; f < T::NQF; ++f) kread[f] = qr * T::KROW + (((2 * f + half) ^ (qr & 7)) * 16);
#pragma unroll
  for (int a = 0; a < 4; ++a) vread[a] = qr * T::VROW + (((2 * a + half) ^ (qr & 7)) * 16);
  CopyPlan<D, B> plan;
  plan.init(wave, lane);

  f32x16 oacc[T::NDT];
#pragma unroll
  for (int i = 0; i < T::NDT; ++i) oacc[i] = f32x16{};
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
      const uint64_t bal = __builtin_amdgcn_ballot_w64(slot >= 0);
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

    // Stages go to the two LDS buffers alternately; the loop body covers one stage in each so that
    // every buffer access has a fixed base.
    const int nstage = total * T::NST;
    auto code_of = [&](int st) { return __builtin_amdgcn_readfirstlane(sList[st / T::NST]); };
    auto lim_of = [&](int code, int st) {
      return (code & 1) ? tail_valid - (st % T::NST) * kStageKeys - 8 * half : kStageKeys;
    };
    if (nstage > 0) plan.issue(pk + (int64_t)(code_of(0) >> 1) * T::SLOT_BYTES, 0, sStage0, wave);
    for (int st = 0; st < nstage; st += 2) {
      // even stage st in buffer 0
      int code = code_of(st);
      wait_vmem();
      __syncthreads();  // stage st visible to all waves; buffer 1 no longer read (stage st - 1 done)
      if (st + 1 < nstage) {
        const int cn = code_of(st + 1);
        plan.issue(pk + (int64_t)(cn >> 1) * T::SLOT_BYTES, (st + 1) % T::NST, sStage1, wave);
      }
      stage_compute<D, B>(sStage0, kread, vread, qf, oacc, m_run, l_run, scale_log2, lim_of(code, st));
      if (st + 1 >= nstage) break;
      // odd stage st + 1 in buffer 1
      code = code_of(st + 1);
      wait_vmem();
      __syncthreads();  // stage st + 1 visible; buffer 0 no longer read
      if (st + 2 < nstage) {
        const int cn = code_of(st + 2);
        plan.issue(pk + (int64_t)(cn >> 1) * T::SLOT_BYTES, (st + 2) % T::NST, sStage0, wave);
      }
      stage_compute<D, B>(sStage1, kread, vread, qf, oacc, m_run, l_run, scale_log2, lim_of(code, st + 1));
    }
    __syncthreads();  // sList and the stage buffers are reused by the next pass
  }

  const float l_tot = sum_halves(l_run);
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
