// Demand union (Eq. 2 of the SparSP paper, section 4.1, kept per head as section 5.2 requires) and its
// compaction into packed slots enumerated by (source rank, head, block) in row-major order (section 5.2,
// metadata-free exchange).  Both kernels are integer-only, atomic-free and deterministic.
#include "sparsp_internal.h"

namespace sparsp {
namespace {

constexpr int kUnionThreads = 1024;     // 64 row groups: enough loads in flight for tall masks
constexpr int kUnionCols = 256;           // mask columns per workgroup = 4 demand words
constexpr int kUnionColGroups = 16;       // 16-byte column groups per workgroup row
constexpr int kUnionRowGroups = kUnionThreads / kUnionColGroups;

// OR of the rank's mask rows for one head and 256 columns.  Each thread streams 16-byte vectors down
// one column group (rows strided by the 64 row groups), the row groups are OR-reduced through LDS, and one
// wave turns the 256 bytes into four 64-bit demand words with ballots (1024 threads: 9-14 % faster than 256
// on 121 and 384 rows).
__global__ __launch_bounds__(kUnionThreads) void union_kernel(const uint8_t* __restrict__ mask, int64_t pitch,
                                                              int Lq, int nb, int W,
                                                              uint64_t* __restrict__ demand) {
  __shared__ uint4 part[kUnionRowGroups][kUnionColGroups];
  __shared__ __align__(16) uint8_t ored[kUnionCols];

  const int h = blockIdx.y;
  const int col0 = blockIdx.x * kUnionCols;
  const int t = threadIdx.x;
  const int cg = t % kUnionColGroups;
  const int rg = t / kUnionColGroups;
  const int col = col0 + cg * 16;

  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  if (col < pitch) {  // pitch is a multiple of 16, so the whole vector lies inside the row
    const uint8_t* p = mask + (int64_t)h * Lq * pitch + col;
    for (int row = rg; row < Lq; row += kUnionRowGroups) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + (int64_t)row * pitch);
      acc.x |= v.x;
      acc.y |= v.y;
      acc.z |= v.z;
      acc.w |= v.w;
    }
  }
  part[rg][cg] = acc;
  __syncthreads();
  if (t < kUnionColGroups) {
    uint4 a = part[0][t];
#pragma unroll
    for (int r = 1; r < kUnionRowGroups; ++r) {
      const uint4 v = part[r][t];
      a.x |= v.x;
      a.y |= v.y;
      a.z |= v.z;
      a.w |= v.w;
    }
    *reinterpret_cast<uint4*>(&ored[t * 16]) = a;
  }
  __syncthreads();
  if (t < 64) {
#pragma unroll
    for (int q = 0; q < kUnionCols / 64; ++q) {
      const int c = col0 + q * 64 + t;
      const uint64_t word = __ballot(c < nb && ored[q * 64 + t] != 0);
      const int w = blockIdx.x * (kUnionCols / 64) + q;
      if (t == 0 && w < W) demand[(int64_t)h * W + w] = word;
    }
  }
}

// One workgroup per head h.  Every workgroup rebuilds the owner bitsets own[p][w] (bit i set when block
// 64w+i belongs to rank p) with ballots, counts the demanded blocks of every (p, h'), and scans the
// counts in (p, h') row-major order; workgroup 0 publishes that scan as seg_offsets.  It then numbers its
// own head's demanded blocks: the slot of block j owned by p is the segment start of (p, h), plus the
// demanded blocks of p in earlier words, plus those below j in the same word.
constexpr int kCompactThreads = 1024;  // 16 waves: owner bitsets and slot numbering over more words at once

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const int32_t* __restrict__ placement, const uint64_t* __restrict__ demand, int H, int G, int nb, int W,
    int32_t* __restrict__ seg_offsets, int32_t* __restrict__ slot_block, int32_t* __restrict__ slot_head,
    int32_t* __restrict__ slot_of) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* own = reinterpret_cast<uint64_t*>(smem);     // [G][W]
  int32_t* pref = reinterpret_cast<int32_t*>(own + G * W);  // [G][W] for this head
  int32_t* cnt = pref + G * W;                              // [G*H + 1], scanned in place

  const int h = blockIdx.x;
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int nwaves = blockDim.x / 64;
  const int GH = G * H;

  for (int w = wave; w < W; w += nwaves) {
    const int j = w * 64 + lane;
    const int p = j < nb ? placement[j] : -1;
    for (int q = 0; q < G; ++q) {
      const uint64_t m = __ballot(p == q);
      if (lane == 0) own[q * W + w] = m;
    }
  }
  __syncthreads();

  for (int t = threadIdx.x; t < GH; t += blockDim.x) {
    const int p = t / H, hh = t - p * H;
    const uint64_t* dw = demand + (int64_t)hh * W;
    const uint64_t* ow = own + p * W;
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popcll(dw[w] & ow[w]);
    cnt[t] = c;
  }
  for (int p = threadIdx.x; p < G; p += blockDim.x) {
    const uint64_t* dw = demand + (int64_t)h * W;
    const uint64_t* ow = own + p * W;
    int run = 0;
    for (int w = 0; w < W; ++w) {
      pref[p * W + w] = run;
      run += __popcll(dw[w] & ow[w]);
    }
  }
  __syncthreads();

  if (wave == 0) {  // exclusive scan of cnt[0, GH): contiguous runs per lane, then a wave scan
    const int per = (GH + 63) / 64;
    const int lo = min(lane * per, GH), hi = min(lo + per, GH);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += cnt[i];
    int incl = s;
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    int run = incl - s;
    for (int i = lo; i < hi; ++i) {
      const int c = cnt[i];
      cnt[i] = run;
      run += c;
    }
    if (lane == 63) cnt[GH] = incl;
  }
  __syncthreads();

  if (h == 0)
    for (int t = threadIdx.x; t <= GH; t += blockDim.x) seg_offsets[t] = cnt[t];

  const uint64_t* dh = demand + (int64_t)h * W;
  for (int w = wave; w < W; w += nwaves) {
    const int j = w * 64 + lane;
    if (j >= nb) continue;
    const uint64_t dw = dh[w];
    const int p = placement[j];
    int32_t s = -1;
    if (((dw >> lane) & 1ull) && p >= 0 && p < G) {
      const uint64_t m = own[p * W + w] & dw;
      s = cnt[p * H + h] + pref[p * W + w] + __popcll(m & ((1ull << lane) - 1ull));
      slot_block[s] = j;
      slot_head[s] = h;
    }
    slot_of[(int64_t)h * nb + j] = s;
  }
}

}  // namespace

hipError_t launch_union(const Dims& g, const uint8_t* mask, int64_t pitch, uint64_t* demand,
                        hipStream_t stream) {
  const dim3 grid((g.W * 64 + kUnionCols - 1) / kUnionCols, g.H);
  hipLaunchKernelGGL(union_kernel, grid, dim3(kUnionThreads), 0, stream, mask, pitch, g.Lq, g.nb, g.W, demand);
  return hipGetLastError();
}

hipError_t launch_compact(const Dims& g, const int32_t* placement, const uint64_t* demand,
                          int32_t* seg_offsets, int32_t* slot_block, int32_t* slot_head, int32_t* slot_of,
                          hipStream_t stream) {
  const size_t lds = compact_lds_bytes(g);
  hipLaunchKernelGGL(compact_kernel, dim3(g.H), dim3(kCompactThreads), lds, stream, placement, demand, g.H, g.G,
                     g.nb, g.W, seg_offsets, slot_block, slot_head, slot_of);
  return hipGetLastError();
}

}  // namespace sparsp
