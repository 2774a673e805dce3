// Pack of the demanded K/V blocks into the compacted buffer (SparSP paper, sections 5.1 and 6.1: only the
// blocks a consumer selected travel, one contiguous region per source rank; section 6.2: arrived blocks
// are placed in the attention kernel's layout).  Slot s = (h, j) receives the K block token-major
// (b x d) followed by the V block transposed (d x b), so the attention kernel's P V product reads
// key-contiguous V rows.  The copy is HBM-bound: every byte is read once and written once with 16-byte
// vector accesses; the V transpose happens in registers on 8 x 8 sub-tiles (the LDS the launch reserves is
// never touched: it only limits how many workgroups a CU holds).
#include "sparsp_internal.h"

namespace sparsp {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackXcdChunk = 16;  // consecutive workgroups (slots) kept on one XCD
// One pack workgroup per CU: the launch reserves more than half of a CU's 160 KiB of LDS (the kernel uses
// none), so a CU holds one 4-wave workgroup instead of seven.  Fewer concurrent streams of DRAM pages
// move the same bytes faster: measured 4.4 % (HunyuanVideo-shaped), 6.3 % (Wan) and 7.8 % (LTX) faster than
// seven per CU; two or three per CU gained only 1.5-2 %, and a persistent grid of one workgroup per CU
// looping over the slots was 5-10 % slower than either.
constexpr size_t kPackLdsReserve = 96 * 1024;
constexpr bool kNtLoad = false;   // K and V are read once
constexpr bool kNtStore = false;  // the packed buffer is written once

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  if (kNtLoad) return __builtin_nontemporal_load(q);
  return *q;
}

__device__ __forceinline__ void store16(uint16_t* p, const u32x4& v) {
  u32x4* q = reinterpret_cast<u32x4*>(p);
  if (kNtStore)
    __builtin_nontemporal_store(v, q);
  else
    *q = v;
}

// Transpose an 8 x 8 tile of 16-bit values held as 8 rows of 4 x 32-bit words (two values per word,
// lower column in the low half).  Output row e holds input column e.
__device__ __forceinline__ void transpose8x8(const uint32_t (&in)[8][4], uint32_t (&out)[8][4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = in[2 * q][e / 2], b = in[2 * q + 1][e / 2];
      out[e][q] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

template <int D, int B>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V,
                                                            const int32_t* __restrict__ seg_offsets, int GH,
                                                            const int32_t* __restrict__ slot_block,
                                                            const int32_t* __restrict__ slot_head,
                                                            int slot_capacity, int H, int nb,
                                                            uint16_t* __restrict__ packed) {
  constexpr int kSub = (B / 8) * (D / 8);         // 8 x 8 sub-tiles per block
  constexpr int kSlotsPerWg = kPackThreads / kSub;  // 1, 2 or 4
  constexpr int kChunksPerThread = 8;               // 16-byte K chunks per thread = (B*D/8) / kSub
  static_assert(kSub * kSlotsPerWg == kPackThreads, "tile shape");
  constexpr int64_t kSlotElems = 2ll * B * D;

  const int S = min(seg_offsets[GH], slot_capacity);
  // Workgroups are dealt to the XCDs in chunks of consecutive slots, so each XCD's L2 sees runs of
  // neighbouring source blocks and output lines (measured 0.6-2.7 % faster than plain round robin).
  const int s = xcd_chunked<kPackXcdChunk>(blockIdx.x) * kSlotsPerWg + threadIdx.x / kSub;
  if (s >= S) return;
  const int u = threadIdx.x % kSub;
  const int h = slot_head[s], j = slot_block[s];
  if ((unsigned)h >= (unsigned)H || (unsigned)j >= (unsigned)nb) return;  // inconsistent slot arrays: skip the slot
  const int64_t src = ((int64_t)h * nb + j) * B * D;
  uint16_t* dst = packed + (int64_t)s * kSlotElems;

  // K: a straight copy; consecutive threads move consecutive 16-byte chunks.
  u32x4 kv[kChunksPerThread];
#pragma unroll
  for (int i = 0; i < kChunksPerThread; ++i) kv[i] = load16(K + src + (int64_t)(u + i * kSub) * 8);

  // V: sub-tile (g, c) = keys 8g..8g+7, columns 8c..8c+7.  Consecutive threads take consecutive key
  // groups g of the same column chunks, so each store instruction of a wave writes whole V^T rows
  // (B keys) and every output line is written by one wave at once.
  const int g = u % (B / 8), c = u / (B / 8);
  uint32_t vin[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 v = load16(V + src + (int64_t)(g * 8 + i) * D + c * 8);
    vin[i][0] = v.x;
    vin[i][1] = v.y;
    vin[i][2] = v.z;
    vin[i][3] = v.w;
  }

#pragma unroll
  for (int i = 0; i < kChunksPerThread; ++i) store16(dst + (int64_t)(u + i * kSub) * 8, kv[i]);

  uint32_t vout[8][4];
  transpose8x8(vin, vout);
  uint16_t* vt = dst + (int64_t)B * D;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const u32x4 o = {vout[e][0], vout[e][1], vout[e][2], vout[e][3]};
    store16(vt + (int64_t)(c * 8 + e) * B + g * 8, o);
  }
}

template <int D, int B>
hipError_t launch_pack_t(const Dims& g, const uint16_t* K, const uint16_t* V, const int32_t* seg_offsets,
                         const int32_t* slot_block, const int32_t* slot_head, int32_t slot_capacity,
                         uint16_t* packed, hipStream_t stream) {
  constexpr int kSlotsPerWg = kPackThreads / ((B / 8) * (D / 8));
  const int64_t hnb = (int64_t)g.H * g.nb;  // S never exceeds H*nb
  const int64_t cap = slot_capacity < hnb ? (int64_t)slot_capacity : hnb;
  constexpr int64_t round = (int64_t)kXcds * kPackXcdChunk;  // whole chunk rounds: the remap is a bijection
  const unsigned grid = (unsigned)(((cap + kSlotsPerWg - 1) / kSlotsPerWg + round - 1) / round * round);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((pack_kernel<D, B>), dim3(grid), dim3(kPackThreads), kPackLdsReserve, stream, K, V,
                     seg_offsets, g.G * g.H, slot_block, slot_head, (int)cap, g.H, g.nb, packed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const Dims& g, const uint16_t* K, const uint16_t* V, const int32_t* seg_offsets,
                       const int32_t* slot_block, const int32_t* slot_head, int32_t slot_capacity,
                       uint16_t* packed, hipStream_t stream) {
  if (g.d == 128 && g.b == 128)
    return launch_pack_t<128, 128>(g, K, V, seg_offsets, slot_block, slot_head, slot_capacity, packed, stream);
  if (g.d == 64 && g.b == 64)
    return launch_pack_t<64, 64>(g, K, V, seg_offsets, slot_block, slot_head, slot_capacity, packed, stream);
  if (g.d == 128 && g.b == 64)
    return launch_pack_t<128, 64>(g, K, V, seg_offsets, slot_block, slot_head, slot_capacity, packed, stream);
  return launch_pack_t<64, 128>(g, K, V, seg_offsets, slot_block, slot_head, slot_capacity, packed, stream);
}

}  // namespace sparsp
