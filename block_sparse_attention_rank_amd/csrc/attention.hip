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
// Pipeline.  Every selected key block is consumed in stages of 64 keys (32 at d = 128, b = 64; see
// stage_keys).  A stage (its K rows and the matching columns of V^T) is copied from global memory straight
// into LDS with global_load_lds_dwordx4 (no register staging); the next stage's copy is issued before the
// current one is computed, into the other of two LDS buffers, and two or more workgroups share a CU.  The
// work is cut into units of 32 keys.  At d = 128 a unit issues the next unit's score MFMAs beside its own
// softmax and then its P V product, with two barriers per 64-key stage (one per 32-key stage).  At d = 64,
// where the softmax costs twice as much per MFMA flop, each unit's P V product is delayed to the next unit
// so that both products' MFMAs sit beside the softmax arithmetic in one stretch of code, with one barrier
// per stage (measured: 5-11 % faster at d = 64, 5 % slower at d = 128, where it needs all 256 VGPRs).  LDS
// rows are
// XOR-swizzled in 16-byte chunks (chunk c of row m sits at c ^ swizzle(m)).  A 16-byte fragment read
// is served 16 lanes at a time by 64 four-byte banks (256 bytes per clock), and its lanes read one
// logical chunk of 16 consecutive rows, so the key gives those rows distinct bank groups; it also keeps
// any 8 consecutive rows apart.  Each lane's fragment addresses are fixed per kernel; the buffer, key
// group and d tile are immediate offsets.
//
// Softmax.  Probabilities are taken against a running maximum that is only raised when needed: they may
// grow to 2^64 before the state is rescaled, which is exact in real arithmetic (numerator and
// denominator share the maximum) and safe in fp32 and bf16.  A unit's row sums reveal when that bound
// is passed (or a row has no maximum yet); only then is the unit's maximum taken, so the common path
// has neither a maximum nor a cross-lane step: the two halves of a row exchange maxima
// (v_permlane32_swap) only when the maximum moves, and their partial sums once at the end.  The
// numerator (the P V product) takes the probabilities rounded to bf16, the denominator adds their fp32
// values: the two differ by the bf16 rounding of each probability (relative 2^-9 at most), well inside the
// output tolerance.
#include <math.h>

#include "sparsp_internal.h"

namespace sparsp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) const void lds_void;

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

// XOR key of the 16-byte chunks of an LDS row of `RowBytes` bytes (256: d = 128 K rows; 128: d = 64 K rows
// and the V^T rows of a 64-key stage; 64: the V^T rows of a 32-key stage).  A 256-byte row covers all 64
// banks, so 16 consecutive rows need 16 distinct keys; two 128-byte rows share the banks, so rows of equal
// parity among 16 need distinct keys, and so do 8 consecutive rows; four 64-byte rows share the banks, so
// rows r, r + 4, r + 8 and r + 12 need distinct keys.
template <int RowBytes>
__device__ __forceinline__ int swizzle(int row) {
  static_assert(RowBytes == 64 || RowBytes == 128 || RowBytes == 256, "row size");
  if constexpr (RowBytes == 64) return (row >> 2) & 3;
  return RowBytes == 256 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

// One LDS-direct copy: every lane moves the 16 bytes at base + voff into LDS at lds + 16 * lane
// (global_load_lds_dwordx4; `lds` is wave-uniform and goes to M0).  It is issued from inline asm so that
// the compiler does not track it: its own tracking of such copies is coarse and would wait for every
// copy in flight before the next LDS read.  The pipeline below orders the copies itself (block_sync),
// and no copy targets a buffer that is read before the barrier that follows its completion.  The s_nop
// covers the wait state between the M0 write and the copy.
__device__ __forceinline__ void copy16(const char* base, uint32_t voff, const unsigned char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const lds_void*)lds;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// Keys per pipeline stage: 64, or 32 at d = 128, b = 64.  That shape's workgroup has two waves; with 64-key
// double buffers of K and V^T (64 KiB) only two workgroups fit a CU, one wave per SIMD, and the compiler then
// spends 292 registers a wave.  With 32-key stages (32 KiB) four fit, two waves per SIMD, in 197 registers:
// measured 17 % faster on a HunyuanVideo-shaped share with 64-token blocks.  At d = 64, b = 64 the same change
// (three waves per SIMD) was 11 % slower, and d = 128, b = 128 already holds two waves per SIMD.
template <int D, int B>
constexpr int stage_keys() {
  return (D == 128 && B == 64) ? 32 : 64;
}
constexpr int kXcdChunk = 16;      // consecutive (head, query block) items kept on one XCD
constexpr int kListCols = 4;       // mask columns a thread reads per listing step (one 32-bit load)

template <int D, int B>
struct Tile {
  static constexpr int NW = B / 32;                      // waves, 32 query rows each
  static constexpr int NT = NW * 64;                     // threads
  static constexpr int SK = stage_keys<D, B>();          // keys per stage
  static constexpr int NST = B / SK;                     // stages per key block
  static constexpr int KROW = D * 2;                     // bytes per K row of a stage
  static constexpr int KBYTES = SK * KROW;               // K part of a stage buffer
  static constexpr int VROW = SK * 2;                    // bytes per V^T row of a stage (128 or 64)
  static constexpr int STAGE = KBYTES + D * VROW;        // one stage buffer
  static constexpr int CH = SK * D / 8;                  // 16-byte chunks of K (and of V^T) per stage
  static constexpr int CPT = CH / NT;                    // K (and V^T) chunks per thread per stage
  static constexpr int NDT = D / 32;                     // 32-row tiles of O^T
  static constexpr int NQF = D / 16;                     // Q fragments along d
  static constexpr int64_t SLOT_BYTES = 4ll * B * D;     // bytes per packed slot
  // Selected blocks listed per pass over the mask row: room for two listing steps, except at d = 64,
  // b = 128, where one step's worth keeps four workgroups within a CU's 160 KiB of LDS.
  static constexpr int LIST = (D == 64 && B == 128) ? kListCols * NT : 2 * kListCols * NT;
  static_assert(CH % NT == 0, "stage must split evenly over the threads");
  static_assert(NT * 16 == 64 * 16 * NW, "one 1 KiB LDS span per wave and copy");
  static_assert(2 * STAGE <= 65536, "LDS offsets must fit the 16-bit immediate");
};

// Stage-invariant parts of this lane's copies.  Copy i of wave w fills LDS chunks (i*NW + w)*64 + lane,
// 16 bytes per lane, of a K buffer and of a V^T buffer.
template <int D, int B>
struct CopyPlan {
  using T = Tile<D, B>;
  uint32_t koff[T::CPT];  // byte offset inside the slot's K part (stage 0)
  uint32_t voff[T::CPT];  // byte offset inside the slot (V^T part, stage 0)

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) {
      const int q = (i * T::NW + wave) * 64 + lane;
      // K: LDS row m, chunk position cp holds logical chunk cp ^ swizzle(m) of key sigma(m).
      const int m = q / (D / 8), cp = q % (D / 8);
      const int c = cp ^ swizzle<T::KROW>(m);
      const int key = (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
      koff[i] = (uint32_t)(key * (D * 2) + c * 16);
      // V^T: LDS row e (a d index), chunk position cp holds keys 8 * (cp ^ swizzle(e)) .. +7.
      const int e = q / (T::SK / 8), vp = q % (T::SK / 8);
      const int vc = vp ^ swizzle<T::VROW>(e);
      voff[i] = (uint32_t)(B * D * 2 + e * (B * 2) + vc * 16);
    }
  }

  // Copy the K rows of stage hh of the slot at `slot` into the LDS buffer `kbuf`.
  __device__ __forceinline__ void issue_k(const char* slot, int hh, unsigned char* kbuf, int wave) const {
    const char* k = slot + hh * T::KBYTES;
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) copy16(k, koff[i], kbuf + (i * T::NW + wave) * 1024);
  }

  // Copy the V^T columns of stage hh of the slot at `slot` into the LDS buffer `vbuf`.
  __device__ __forceinline__ void issue_v(const char* slot, int hh, unsigned char* vbuf, int wave) const {
    const char* v = slot + hh * T::VROW;
#pragma unroll
    for (int i = 0; i < T::CPT; ++i) copy16(v, voff[i], vbuf + (i * T::NW + wave) * 1024);
  }
};

// Per-lane state of the online softmax and the output accumulator.
template <int D, int B>
struct RowState {
  using T = Tile<D, B>;
  f32x16 oacc[T::NDT];
  float m_run;  // maximum the probabilities are taken against (log2-scaled logits)
  float l_run;  // sum of this lane's fp32 probabilities relative to m_run (the P V product takes them rounded to bf16)
};

// A unit is one 32-key group g of a stage.  Its scores S^T = K Q^T come from one MFMA tile:
// sacc[4i + r] is key 32g + 16(i >> 1) + 8 half + 4(i & 1) + r of the stage for query row lane % 32
// (the K rows sit in LDS in that permuted order).
template <int D, int B>
__device__ __forceinline__ f32x16 unit_scores(const unsigned char* kbuf, int g, const uint32_t (&kread)[Tile<D, B>::NQF],
                                              const bf16x8 (&qf)[Tile<D, B>::NQF]) {
  using T = Tile<D, B>;
  f32x16 sacc = f32x16{};
#pragma unroll
  for (int f = 0; f < T::NQF; ++f)
    sacc = mfma32(*reinterpret_cast<const bf16x8*>(kbuf + kread[f] + g * 32 * T::KROW), qf[f], sacc);
  return sacc;
}

// Mask the padding keys of the last block in a unit's scores: key offsets at or past `lim` inside the
// unit, counted from 8 half (lim >= 24 masks nothing).
__device__ __forceinline__ void unit_mask(f32x16& sacc, int lim) {
  if (lim < 32) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int c = 16 * (x / 8) + 4 * ((x / 4) % 2) + (x % 4);
      if (c >= lim) sacc[x] = -INFINITY;
    }
  }
}

// Probabilities of a unit, rounded to bf16 for the second product; returns the sum of their fp32 values
// (two add chains, each seeded with its first term: p >= +0, so this equals a sum started from zero
// without the two additions of zero the compiler would have to keep).  pf[b] holds keys 16b + 8 half +
// 0..7 of the unit.  (A v_dot2 against (1, 1) would sum the rounded pairs in half the instructions, but
// on gfx950 it competes with the MFMAs of the other wave on the SIMD and issues several times slower
// than two adds.)
__device__ __forceinline__ float unit_probabilities(const f32x16& sacc, float scale_log2, float m_run, bf16x8 (&pf)[2]) {
  float p[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    p[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[x], scale_log2, -m_run));
    pf[x / 8][x % 8] = (__bf16)p[x];
  }
  float l_even = p[0], l_odd = p[1];
#pragma unroll
  for (int x = 2; x < 16; x += 2) {
    l_even += p[x];
    l_odd += p[x + 1];
  }
  return l_even + l_odd;
}

// O^T += V^T P^T for unit g: step b covers keys 32g + 16b + 8 half + 0..7 of the stage, one V^T fragment.
template <int D, int B>
__device__ __forceinline__ void unit_accumulate(const unsigned char* vbuf, int g, const uint32_t (&vread)[4],
                                                const bf16x8 (&pf)[2], f32x16 (&oacc)[Tile<D, B>::NDT]) {
  using T = Tile<D, B>;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < T::NDT; ++i)
      oacc[i] = mfma32(*reinterpret_cast<const bf16x8*>(vbuf + vread[2 * g + b] + i * 32 * T::VROW), pf[b], oacc[i]);
}

// The rare path of a unit's softmax.  Probabilities are first taken against the running maximum without a
// per-unit maximum: they may reach 2^64 (exact in fp32 and bf16, and the fp32 sums stay far from overflow).
// The lane's 16-key sum, which the row sum needs anyway, tells whether any probability went past 2^64 (or is
// inf or NaN: the first unit of a row, whose maximum is still -inf); only then is this called: it takes the
// unit's maximum, rescales the state (the accumulator already holds every earlier unit, including the one
// whose P V product was issued in this unit, all relative to the old maximum) and recomputes the unit's
// probabilities.
template <int D, int B>
__device__ __forceinline__ void unit_rescale(const f32x16& sacc, RowState<D, B>& rs, float scale_log2,
                                                       bf16x8 (&pf)[2], float& lu) {
  using T = Tile<D, B>;
  float mx = -INFINITY;
#pragma unroll
  for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[x]);
  const float m_new = fmaxf(rs.m_run, max_halves(mx * scale_log2));  // scale_log2 > 0
  if (m_new != -INFINITY) {  // -inf: no key of the row seen yet; nothing to rescale
    const float alpha = rs.m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rs.m_run - m_new);
    rs.m_run = m_new;
    rs.l_run *= alpha;
#pragma unroll
    for (int i = 0; i < T::NDT; ++i) rs.oacc[i] *= alpha;
  }
  lu = unit_probabilities(sacc, scale_log2, m_new == -INFINITY ? 0.f : m_new, pf);
}

// Softmax of a unit whose P V product follows at once (the d = 128 schedule).
template <int D, int B>
__device__ __forceinline__ void unit_softmax(const f32x16& sacc, RowState<D, B>& rs, float scale_log2, bf16x8 (&pf)[2]) {
  float lu = unit_probabilities(sacc, scale_log2, rs.m_run, pf);
  if (__builtin_amdgcn_ballot_w64(!(lu < 0x1p64f)) != 0) unit_rescale<D, B>(sacc, rs, scale_log2, pf, lu);
  rs.l_run += lu;
}

// Workgroup barrier for the stage pipeline: wait until at most `NOut` of this lane's vector memory
// operations (the LDS-direct copies) are outstanding and its LDS reads have returned, then s_barrier.
// __syncthreads() would also wait for the copies still meant to be in flight.  As one volatile asm
// statement with a memory clobber it is also a hard scheduling fence, so no LDS access moves across it
// (the compiler does not model the LDS write of a direct copy).
template <int NOut>
__device__ __forceinline__ void block_sync() {
  static_assert(NOut >= 0 && NOut < 64, "vmcnt field");
  // s_waitcnt immediate: vmcnt bits 3:0 and 15:14, expcnt 6:4 (7: no wait), lgkmcnt 11:8 (0).
  __builtin_amdgcn_s_waitcnt((NOut & 15) | ((NOut >> 4) << 14) | 0x0070);
  asm volatile("s_barrier" ::: "memory");
}

// Exclusive prefix, in thread order, of a per-thread count in 0..4 over the workgroup, and the workgroup's
// total.  Two barriers; sWaveCnt holds one int per wave.
template <int NW>
__device__ __forceinline__ int block_prefix4(int cnt, int lane, int wave, int* sWaveCnt, int& total) {
  int below = 0, wave_total = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t bal = __builtin_amdgcn_ballot_w64((cnt >> bit) & 1);
    below += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)) << bit;
    wave_total += __popcll(bal) << bit;
  }
  if (lane == 0) sWaveCnt[wave] = wave_total;
  __syncthreads();
  int off = below;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = sWaveCnt[w];
    off += w < wave ? c : 0;
    total += c;
  }
  __syncthreads();
  return off;
}

// Column of the median selected block of a mask row: the floor(count / 2)-th selected column in ascending
// order (0 for an empty row).  Threads read kListCols consecutive mask bytes per step with one 32-bit load.
template <int NT, int NW>
__device__ int median_column(const uint8_t* mrow, int nb, int t, int lane, int wave, int* sWaveCnt, int* sOut) {
  auto selected = [&](int j0, int& cnt) {
    const uint32_t w = j0 < nb ? *reinterpret_cast<const uint32_t*>(mrow + j0) : 0u;
    uint32_t bits = 0;
#pragma unroll
    for (int c = 0; c < kListCols; ++c) bits |= (j0 + c < nb && ((w >> (8 * c)) & 0xffu) != 0u) ? (1u << c) : 0u;
    cnt = __popc(bits);
    return bits;
  };
  int count = 0;
  for (int col = 0; col < nb; col += kListCols * NT) {
    int cnt, tot;
    selected(col + kListCols * t, cnt);
    block_prefix4<NW>(cnt, lane, wave, sWaveCnt, tot);
    count += tot;
  }
  const int target = count / 2;
  if (t == 0) *sOut = 0;
  int base = 0;
  for (int col = 0; col < nb && base <= target; col += kListCols * NT) {
    const int j0 = col + kListCols * t;
    int cnt, tot;
    uint32_t bits = selected(j0, cnt);
    const int off = base + block_prefix4<NW>(cnt, lane, wave, sWaveCnt, tot);
    if (target >= off && target < off + cnt) {
      for (int r = target - off; r > 0; --r) bits &= bits - 1;  // drop the lower selected columns
      *sOut = j0 + __builtin_ctz(bits);
    }
    base += tot;
  }
  __syncthreads();
  const int J = *sOut;
  __syncthreads();
  return J;
}

template <int D, int B>
__global__ __launch_bounds__(2 * B) __attribute__((amdgpu_waves_per_eu(2, 2))) void bsa_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ mask, int64_t pitch,
    const int32_t* __restrict__ slot_of, const uint16_t* __restrict__ packed, int slot_lo, int slot_hi, float scale_log2,
    int h_lo, int n_heads, int Lq, int nb, int N, float* __restrict__ O, float* __restrict__ lse, int accumulate,
    int anchored) {
  using T = Tile<D, B>;
  // Separate double buffers for K and V^T.  The work is cut into units of 32 keys (two per stage); the
  // scores of unit u + 1 are computed while unit u is turned into probabilities, and then unit u is
  // accumulated, so K runs half a stage ahead of V.
  __shared__ __align__(1024) unsigned char sK0[T::KBYTES];
  __shared__ __align__(1024) unsigned char sK1[T::KBYTES];
  __shared__ __align__(1024) unsigned char sV0[D * T::VROW];
  __shared__ __align__(1024) unsigned char sV1[D * T::VROW];
  __shared__ int sList[T::LIST];
  __shared__ int sWaveCnt[T::NW];
  __shared__ int sAnchor, sRot;

  const int wid = xcd_chunked<kXcdChunk>(blockIdx.x);
  if (wid >= n_heads * Lq) return;  // padding of the grid to whole chunk rounds
  const int hh = wid / Lq, k = wid - hh * Lq;
  const int h = h_lo + hh;
  const int t = threadIdx.x, lane = t % 64;
  const int wave = __builtin_amdgcn_readfirstlane(t / 64);
  const int qr = lane % 32, half = lane / 32;

  // Q^T fragments (B operand of S^T = K Q^T): row qr of this wave, d = 16f + 8*half .. +7.
  const int64_t row = (int64_t)h * Lq * B + (int64_t)k * B + wave * 32 + qr;
  bf16x8 qf[T::NQF];
#pragma unroll
  for (int f = 0; f < T::NQF; ++f) qf[f] = *reinterpret_cast<const bf16x8*>(Q + row * D + f * 16 + half * 8);

  // This lane's LDS fragment addresses inside a buffer.  Every row it reads is qr plus a multiple of 32,
  // so one swizzle key serves all of them.
  uint32_t kread[T::NQF], vread[4];
#pragma unroll
  for (int f = 0; f < T::NQF; ++f) kread[f] = qr * T::KROW + (((2 * f + half) ^ swizzle<T::KROW>(qr)) * 16);
#pragma unroll
  for (int a = 0; a < 4; ++a)  // 16-key steps of a stage: 4 at 64 keys, 2 at 32 (the rest unused)
    vread[a] = a < T::SK / 16 ? qr * T::VROW + (((2 * a + half) ^ swizzle<T::VROW>(qr)) * 16) : 0u;
  CopyPlan<D, B> plan;
  plan.init(wave, lane);

  RowState<D, B> rs;
#pragma unroll
  for (int i = 0; i < T::NDT; ++i) rs.oacc[i] = f32x16{};
  rs.m_run = -INFINITY;
  rs.l_run = 0.f;

  // d = 64 schedule: the V^T buffers start at zero so that the first unit's empty pending product (0 x
  // finite) adds nothing.
  if constexpr (D == 64)
    for (int i = t * 16; i < 2 * D * T::VROW; i += T::NT * 16)
      *reinterpret_cast<uint4*>((i < D * T::VROW ? sV0 : sV1) + (i % (D * T::VROW))) = make_uint4(0u, 0u, 0u, 0u);
  bf16x8 pfp[2];  // d = 64 schedule: probabilities of the unit whose P V product is still pending

  const uint8_t* mrow = mask + ((int64_t)h * Lq + k) * pitch;
  // Order of the stages (b = 128).  Neighbouring query blocks select mostly the same key blocks, each row's
  // set shifted by about one block from the previous row's.  In ascending j a row then reads a shared block
  // one block step after its neighbour, and 64 workgroups per XCD stream 4 MB in a block step, the size of
  // the XCD's L2.  Every row therefore starts its (single-pass) list at a common column and wraps around:
  // the median selected column of the first row of its group of 16 local query blocks, whose items the
  // XCD dealing keeps together.  Neighbours then read their shared blocks at about the same time.  (An LRU
  // model of one XCD's L2 under this dispatch puts the stage copies that hit in L2 at 65 % instead of 50 %
  // at the HunyuanVideo shape, 57 % instead of 49 % at the Wan shape; at b = 64 ascending order is better.)
  // Only the single-pass call orders its stages this way: a segment or chunk launch lists only its piece's
  // few blocks per row, where the order gains little, and skips the anchor's two passes over a mask row.
  int anchor = 0;
  if constexpr (B == 128)
    if (anchored)
      anchor = median_column<T::NT, T::NW>(mask + ((int64_t)h * Lq + (k & ~15)) * pitch, nb, t, lane, wave,
                                           sWaveCnt, &sAnchor);
  const int32_t* sof = slot_of + (int64_t)h * nb;
  const int tail_valid = N - (nb - 1) * B;  // real keys in the last block, 1..B
  const char* pk = reinterpret_cast<const char*>(packed);

  int col = 0;
  int seen = 0;  // selected blocks in the slot range, over all passes
  while (col < nb) {
    const bool first_pass = col == 0;
    if (t == 0) sRot = 0;
    // List the selected blocks of the next columns (ascending j) as (slot << 1 | is_last_block).  A thread
    // reads kListCols consecutive mask bytes with one load (rows are 16-byte aligned and their pitch is a
    // multiple of 16, so the word stays inside the row; columns >= nb are ignored) and looks up their slots;
    // its entries go after those of the lower lanes and waves, whose counts come from one ballot per bit of
    // the per-thread count.
    int total = 0;
    while (col < nb && total <= T::LIST - kListCols * T::NT) {
      const int j0 = col + kListCols * t;
      const uint32_t mbits = j0 < nb ? *reinterpret_cast<const uint32_t*>(mrow + j0) : 0u;
      int slots[kListCols];
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < kListCols; ++c) {
        const int j = j0 + c;
        int slot = -1;
        if (j < nb && ((mbits >> (8 * c)) & 0xffu) != 0u) {
          slot = sof[j];
          if (slot < slot_lo || slot >= slot_hi) slot = -1;  // outside the consumed slot range
        }
        slots[c] = slot;
        cnt += slot >= 0 ? 1 : 0;
      }
      int below = 0, wave_total = 0;  // entries of the lower lanes of this wave; of the whole wave
#pragma unroll
      for (int bit = 0; bit < 3; ++bit) {  // cnt <= 4 < 8
        const uint64_t bal = __builtin_amdgcn_ballot_w64((cnt >> bit) & 1);
        below += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))
                 << bit;
        wave_total += __popcll(bal) << bit;
      }
      if (lane == 0) sWaveCnt[wave] = wave_total;
      __syncthreads();
      int off = total + below, add = 0;
#pragma unroll
      for (int w = 0; w < T::NW; ++w) {
        const int c = sWaveCnt[w];
        off += w < wave ? c : 0;
        add += c;
      }
      int before_anchor = 0;
#pragma unroll
      for (int c = 0; c < kListCols; ++c)
        if (slots[c] >= 0) {
          sList[off++] = (slots[c] << 1) | (j0 + c == nb - 1 ? 1 : 0);
          before_anchor += j0 + c < anchor ? 1 : 0;
        }
      if (before_anchor != 0) atomicAdd(&sRot, before_anchor);
      total += add;
      col += kListCols * T::NT;
      __syncthreads();
    }

    seen += total;
    const int n = total * T::NST;  // stages of this pass
    // Entries before the anchor go last (a row listed in one pass only).
    const int rot = first_pass && col >= nb ? sRot : 0;
    if (n > 0) {
      // Slot code of stage s (clamped to the last stage: codes past the end are only read, never used).
      auto code_of = [&](int s) {
        int e = min(s, n - 1) / T::NST + rot;
        e -= e >= total ? total : 0;
        return __builtin_amdgcn_readfirstlane(sList[e]);
      };
      auto slot_ptr = [&](int code) { return pk + (int64_t)(code >> 1) * T::SLOT_BYTES; };
      // Offset of the first padding key inside unit g of stage s, counted from 8 half (>= 32: none).
      auto lim_of = [&](int code, int s, int g) {
        return (code & 1) ? tail_valid - (s % T::NST) * T::SK - 32 * g - 8 * half : 32;
      };

      if constexpr (T::SK == 32) {
        // 32-key stages, one unit each, P V product at once.  At the top of unit s every lane waits for its copies
        // of K[s + 1] and V^T[s] (issued at the top of unit s - 1) and the workgroup meets, which frees K[s]'s
        // buffer (last read by the lookahead scores of unit s - 1) and V^T[s - 1]'s; K[s + 2] and V^T[s + 1] are
        // issued into them.
        auto unit = [&](f32x16& cur, f32x16& nxt, const unsigned char* kbuf_next, const unsigned char* vbuf, int lim) {
          bf16x8 pf[2];
          unit_mask(cur, lim);
          nxt = unit_scores<D, B>(kbuf_next, 0, kread, qf);
          unit_softmax<D, B>(cur, rs, scale_log2, pf);
          __builtin_amdgcn_s_setprio(1);
          unit_accumulate<D, B>(vbuf, 0, vread, pf, rs.oacc);
          __builtin_amdgcn_s_setprio(0);
        };
        int c0 = code_of(0), c1 = code_of(1), c2 = code_of(2);  // codes of stages s, s + 1, s + 2
        plan.issue_k(slot_ptr(c0), 0, sK0, wave);
        plan.issue_v(slot_ptr(c0), 0, sV0, wave);
        if (n > 1) {
          plan.issue_k(slot_ptr(c1), 1 % T::NST, sK1, wave);
          block_sync<T::CPT>();
        } else {
          block_sync<0>();
        }
        f32x16 sa = unit_scores<D, B>(sK0, 0, kread, qf), sb;
        for (int s = 0; s < n; s += 2) {
          block_sync<0>();
          if (s + 2 < n) plan.issue_k(slot_ptr(c2), (s + 2) % T::NST, sK0, wave);
          if (s + 1 < n) plan.issue_v(slot_ptr(c1), (s + 1) % T::NST, sV1, wave);
          int c3 = code_of(s + 3);
          unit(sa, sb, sK1, sV0, lim_of(c0, s, 0));
          if (s + 1 >= n) break;
          c0 = c1; c1 = c2; c2 = c3;
          block_sync<0>();
          if (s + 3 < n) plan.issue_k(slot_ptr(c2), (s + 3) % T::NST, sK1, wave);
          if (s + 2 < n) plan.issue_v(slot_ptr(c1), (s + 2) % T::NST, sV0, wave);
          c3 = code_of(s + 4);
          unit(sb, sa, sK0, sV1, lim_of(c0, s + 1, 0));
          c0 = c1; c1 = c2; c2 = c3;
        }
      } else if constexpr (D == 64) {
        // One unit u: the scores of unit u + 1, the probabilities of unit u and the P V product of unit u - 1
        // (whose probabilities are already in pfp) are issued together, so the MFMAs of both products sit
        // beside the softmax arithmetic in one stretch of code; the rare rescale follows.  After the last unit
        // the "next" scores read a stale buffer and are dropped.
        auto unit = [&](f32x16& cur, f32x16& nxt, const unsigned char* kbuf_next, int g_next,
                        const unsigned char* vbuf_prev, int g_prev, int lim) {
          bf16x8 pf[2];
          unit_mask(cur, lim);
          nxt = unit_scores<D, B>(kbuf_next, g_next, kread, qf);
          float lu = unit_probabilities(cur, scale_log2, rs.m_run, pf);
          unit_accumulate<D, B>(vbuf_prev, g_prev, vread, pfp, rs.oacc);
          if (__builtin_amdgcn_ballot_w64(!(lu < 0x1p64f)) != 0) unit_rescale<D, B>(cur, rs, scale_log2, pf, lu);
          rs.l_run += lu;
          pfp[0] = pf[0];
          pfp[1] = pf[1];
        };

        // Copies, one barrier per 64-key stage: at the top of unit 2s + 1 every lane waits for all its copies
        // (K[s + 1] and V^T[s], issued one stage earlier) and the workgroup meets, which makes them visible and
        // frees K[s]'s buffer (last read by the scores of unit 2s + 1, issued in unit 2s) and V^T[s - 1]'s
        // (last read by the P V product of unit 2s - 1, issued in unit 2s); K[s + 2] and V^T[s + 1] are then
        // issued into them.  The first unit of a pass carries no pending product (pfp = 0 against a V^T
        // buffer holding finite values).
        int c0 = code_of(0), c1 = code_of(1), c2 = code_of(2);  // codes of stages s, s + 1, s + 2
        pfp[0] = bf16x8{};
        pfp[1] = bf16x8{};
        // The Q fragment loads finished long ago; saying so here keeps the compiler from waiting on them
        // (and with them on the copies issued after them) before the first scores.
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        plan.issue_k(slot_ptr(c0), 0, sK0, wave);
        plan.issue_k(slot_ptr(c1), 1 % T::NST, sK1, wave);
        plan.issue_v(slot_ptr(c0), 0, sV0, wave);
        block_sync<2 * T::CPT>();  // K[0] has landed (copies complete in issue order)
        f32x16 sa = unit_scores<D, B>(sK0, 0, kread, qf), sb;

        for (int s = 0; s < n; s += 2) {
          // stage s (even): K[s] in sK0, K[s + 1] in sK1 and V^T[s] in sV0 landing, V^T[s - 1] in sV1
          int c3 = code_of(s + 3);
          unit(sa, sb, sK0, 1, sV1, 1, lim_of(c0, s, 0));
          block_sync<0>();
          if (s + 2 < n) plan.issue_k(slot_ptr(c2), (s + 2) % T::NST, sK0, wave);
          if (s + 1 < n) plan.issue_v(slot_ptr(c1), (s + 1) % T::NST, sV1, wave);
          unit(sb, sa, sK1, 0, sV0, 0, lim_of(c0, s, 1));
          if (s + 1 >= n) {
            unit_accumulate<D, B>(sV0, 1, vread, pfp, rs.oacc);
            break;
          }
          c0 = c1; c1 = c2; c2 = c3;

          // stage s + 1 (odd): K[s + 1] in sK1, K[s + 2] in sK0 and V^T[s + 1] in sV1 landing, V^T[s] in sV0
          c3 = code_of(s + 4);
          unit(sa, sb, sK1, 1, sV0, 1, lim_of(c0, s + 1, 0));
          block_sync<0>();
          if (s + 3 < n) plan.issue_k(slot_ptr(c2), (s + 3) % T::NST, sK1, wave);
          if (s + 2 < n) plan.issue_v(slot_ptr(c1), (s + 2) % T::NST, sV0, wave);
          unit(sb, sa, sK0, 0, sV1, 0, lim_of(c0, s + 1, 1));
          if (s + 2 >= n) {
            unit_accumulate<D, B>(sV1, 1, vread, pfp, rs.oacc);
            break;
          }
          c0 = c1; c1 = c2; c2 = c3;
        }
      } else {
        // One unit: head of its scores, then the next unit's scores beside its probabilities, then its
        // accumulation.  After the last unit the "next" scores read a stale buffer and are dropped.
        auto unit = [&](f32x16& cur, f32x16& nxt, const unsigned char* kbuf_next, int g_next,
                        const unsigned char* vbuf, int g, int lim) {
          bf16x8 pf[2];
          unit_mask(cur, lim);
          nxt = unit_scores<D, B>(kbuf_next, g_next, kread, qf);
          unit_softmax<D, B>(cur, rs, scale_log2, pf);
          // The P V cluster runs at raised wave priority: the SIMD's other wave is mid-softmax, and
          // letting this wave's MFMAs issue first keeps the matrix pipe fed (measured 3 % faster).
          __builtin_amdgcn_s_setprio(1);
          unit_accumulate<D, B>(vbuf, g, vread, pf, rs.oacc);
          __builtin_amdgcn_s_setprio(0);
        };

        // Copies: V^T[s + 1] is issued at the top of unit 2s (its buffer held V^T[s - 1], last read in unit
        // 2s - 1), K[s + 2] at the top of unit 2s + 1 (its buffer held K[s], last read in unit 2s).  Each
        // top waits for this lane's older copy and then for the whole workgroup, which makes V^T[s] (top of
        // unit 2s) or K[s + 1] (top of unit 2s + 1) visible and frees the buffer it refills; the newer copy
        // (CPT instructions) stays in flight when it was issued.
        int c0 = code_of(0), c1 = code_of(1), c2 = code_of(2);  // codes of stages s, s + 1, s + 2
        plan.issue_k(slot_ptr(c0), 0, sK0, wave);
        plan.issue_v(slot_ptr(c0), 0, sV0, wave);
        block_sync<0>();
        if (n > 1) plan.issue_k(slot_ptr(c1), 1 % T::NST, sK1, wave);
        f32x16 sa = unit_scores<D, B>(sK0, 0, kread, qf), sb;

        for (int s = 0; s < n; s += 2) {
          // stage s (even): K[s] in sK0, V^T[s] in sV0, K[s + 1] in sK1
          if (s + 1 < n) block_sync<T::CPT>(); else block_sync<0>();
          if (s + 1 < n) plan.issue_v(slot_ptr(c1), (s + 1) % T::NST, sV1, wave);
          int c3 = code_of(s + 3);
          unit(sa, sb, sK0, 1, sV0, 0, lim_of(c0, s, 0));
          if (s + 1 < n) block_sync<T::CPT>(); else block_sync<0>();
          if (s + 2 < n) plan.issue_k(slot_ptr(c2), (s + 2) % T::NST, sK0, wave);
          unit(sb, sa, sK1, 0, sV0, 1, lim_of(c0, s, 1));
          if (s + 1 >= n) break;
          c0 = c1; c1 = c2; c2 = c3;

          // stage s + 1 (odd): K[s + 1] in sK1, V^T[s + 1] in sV1, K[s + 2] in sK0
          if (s + 2 < n) block_sync<T::CPT>(); else block_sync<0>();
          if (s + 2 < n) plan.issue_v(slot_ptr(c1), (s + 2) % T::NST, sV0, wave);
          c3 = code_of(s + 4);
          unit(sa, sb, sK1, 1, sV1, 0, lim_of(c0, s + 1, 0));
          if (s + 2 < n) block_sync<T::CPT>(); else block_sync<0>();
          if (s + 3 < n) plan.issue_k(slot_ptr(c2), (s + 3) % T::NST, sK1, wave);
          unit(sb, sa, sK0, 0, sV1, 1, lim_of(c0, s + 1, 1));
          c0 = c1; c1 = c2; c2 = c3;
        }
      }
    }
    __syncthreads();  // sList and the buffers are reused by the next pass
  }

  const float l_tot = sum_halves(rs.l_run);
  const float lse_part = l_tot > 0.f ? rs.m_run * 0.69314718055994531f + logf(l_tot) : -INFINITY;
  float* orow = O + row * D;
  if (accumulate) {
    // Fold this partial result into the running one held in O and lse (the online softmax of whole pieces
    // of KV): lse <- ln(e^lse + e^lse_part), O <- e^(lse_old - lse) O + e^(lse_part - lse) O_part.  An
    // item without any selected block in the range leaves its rows as they are.
    if (seen == 0) return;
    const float lse_old = lse[row];
    const float m = fmaxf(lse_old, lse_part);
    if (m == -INFINITY) return;  // both empty: the row stays (0, -inf) or as it was
    const float w_old = expf(lse_old - m), w_part = expf(lse_part - m);
    const float wsum = w_old + w_part;
    const float a = w_old / wsum;
    const float c = l_tot > 0.f ? (w_part / wsum) / l_tot : 0.f;
#pragma unroll
    for (int i = 0; i < T::NDT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4* dst = reinterpret_cast<float4*>(orow + i * 32 + q * 8 + half * 4);
        const float4 o = *dst;
        *dst = make_float4(a * o.x + c * rs.oacc[i][4 * q + 0], a * o.y + c * rs.oacc[i][4 * q + 1],
                           a * o.z + c * rs.oacc[i][4 * q + 2], a * o.w + c * rs.oacc[i][4 * q + 3]);
      }
    if (half == 0) lse[row] = m + logf(wsum);
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int i = 0; i < T::NDT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = make_float4(rs.oacc[i][4 * q + 0] * inv, rs.oacc[i][4 * q + 1] * inv,
                                   rs.oacc[i][4 * q + 2] * inv, rs.oacc[i][4 * q + 3] * inv);
      *reinterpret_cast<float4*>(orow + i * 32 + q * 8 + half * 4) = v;
    }
  if (half == 0) lse[row] = lse_part;
}

template <int D, int B>
hipError_t launch_attention_t(const Dims& g, const uint16_t* Q, const uint8_t* mask, int64_t pitch,
                              const int32_t* slot_of, const uint16_t* packed, int32_t slot_lo, int32_t slot_hi,
                              int h_lo, int h_hi, float softmax_scale, float* O, float* lse, int accumulate,
                              int anchored, hipStream_t stream) {
  const int64_t items = (int64_t)(h_hi - h_lo) * g.Lq;
  if (items == 0) return hipSuccess;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  constexpr int64_t round = (int64_t)kXcds * kXcdChunk;
  const int64_t grid = (items + round - 1) / round * round;
  hipLaunchKernelGGL((bsa_fwd_kernel<D, B>), dim3((unsigned)grid), dim3(2 * B), 0, stream, Q, mask, pitch,
                     slot_of, packed, slot_lo, slot_hi, scale_log2, h_lo, h_hi - h_lo, g.Lq, g.nb, g.N, O, lse,
                     accumulate, anchored);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const Dims& g, const uint16_t* Q, const uint8_t* mask, int64_t pitch,
                            const int32_t* slot_of, const uint16_t* packed, int32_t slot_lo, int32_t slot_hi,
                            int32_t h_lo, int32_t h_hi, float softmax_scale, float* O, float* lse, int accumulate,
                            int anchored, hipStream_t stream) {
  if (g.d == 128 && g.b == 128)
    return launch_attention_t<128, 128>(g, Q, mask, pitch, slot_of, packed, slot_lo, slot_hi, h_lo, h_hi, softmax_scale,
                                        O, lse, accumulate, anchored, stream);
  if (g.d == 64 && g.b == 64)
    return launch_attention_t<64, 64>(g, Q, mask, pitch, slot_of, packed, slot_lo, slot_hi, h_lo, h_hi, softmax_scale,
                                      O, lse, accumulate, anchored, stream);
  if (g.d == 128 && g.b == 64)
    return launch_attention_t<128, 64>(g, Q, mask, pitch, slot_of, packed, slot_lo, slot_hi, h_lo, h_hi, softmax_scale,
                                       O, lse, accumulate, anchored, stream);
  return launch_attention_t<64, 128>(g, Q, mask, pitch, slot_of, packed, slot_lo, slot_hi, h_lo, h_hi, softmax_scale,
                                     O, lse, accumulate, anchored, stream);
}

}  // namespace sparsp
