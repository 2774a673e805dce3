// The C ABI of libsparsp: argument checks, geometry derivation and kernel launches.  Declarations and the
// contract of every entry point are in include/sparsp.h.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "sparsp.h"
#include "sparsp_internal.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fn, const char* what) {
  char buf[512];
  snprintf(buf, sizeof(buf), "%s: %s", fn, what);
  g_last_error = buf;
  return status;
}

int32_t hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return SPARSP_OK;
  char buf[512];
  snprintf(buf, sizeof(buf), "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  g_last_error = buf;
  return SPARSP_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the geometry shared by every device call; fills `out` on success.
int32_t check_geometry(const sparsp_geometry* g, const char* fn, sparsp::Dims* out) {
  if (!g) return fail(SPARSP_ERR_INVALID, fn, "geometry is NULL");
  if (g->H < 1) return fail(SPARSP_ERR_INVALID, fn, "H must be >= 1");
  if (g->N < 1) return fail(SPARSP_ERR_INVALID, fn, "N must be >= 1");
  if (g->G < 1) return fail(SPARSP_ERR_INVALID, fn, "G must be >= 1");
  if (g->r < 0 || g->r >= g->G) return fail(SPARSP_ERR_INVALID, fn, "r must lie in [0, G)");
  if (g->d != 64 && g->d != 128) return fail(SPARSP_ERR_UNSUPPORTED, fn, "d must be 64 or 128");
  if (g->b != 64 && g->b != 128) return fail(SPARSP_ERR_UNSUPPORTED, fn, "b must be 64 or 128");
  if (g->G > sparsp::kMaxRanks) return fail(SPARSP_ERR_UNSUPPORTED, fn, "G must be <= 64");
  const int64_t nb = ((int64_t)g->N + g->b - 1) / g->b;
  if (nb > sparsp::kMaxBlocks) return fail(SPARSP_ERR_UNSUPPORTED, fn, "nb = ceil(N/b) must be <= 16384");
  if (g->Lq < 0 || g->Lq > nb) return fail(SPARSP_ERR_INVALID, fn, "Lq must lie in [0, nb]");
  if ((int64_t)g->H * nb > (1ll << 30)) return fail(SPARSP_ERR_UNSUPPORTED, fn, "H*nb must be <= 2^30");
  out->H = g->H;
  out->d = g->d;
  out->b = g->b;
  out->N = g->N;
  out->G = g->G;
  out->r = g->r;
  out->Lq = g->Lq;
  out->nb = (int)nb;
  out->W = (int)((nb + 63) / 64);
  return SPARSP_OK;
}

int32_t check_mask(const sparsp::Dims& d, const uint8_t* mask, int64_t pitch, const char* fn) {
  if (!mask && d.Lq > 0) return fail(SPARSP_ERR_INVALID, fn, "mask is NULL");
  if (pitch < d.nb || pitch % 16 != 0) return fail(SPARSP_ERR_INVALID, fn, "mask_pitch must be >= nb and a multiple of 16");
  if (mask && !aligned16(mask)) return fail(SPARSP_ERR_INVALID, fn, "mask must be 16-byte aligned");
  return SPARSP_OK;
}

}  // namespace

extern "C" {

int32_t sparsp_abi_version(void) { return SPARSP_ABI_VERSION; }

const char* sparsp_status_string(int32_t status) {
  switch (status) {
    case SPARSP_OK: return "ok";
    case SPARSP_ERR_INVALID: return "invalid argument";
    case SPARSP_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPARSP_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sparsp_last_error(void) { return g_last_error.c_str(); }

int32_t sparsp_local_query_blocks(const int32_t* placement, int32_t nb, int32_t G, int32_t r, int32_t* q_blocks,
                                  int32_t capacity, int32_t* Lq) {
  static const char* fn = "sparsp_local_query_blocks";
  if (!placement || !Lq) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (nb < 1 || G < 1) return fail(SPARSP_ERR_INVALID, fn, "nb and G must be >= 1");
  if (r < 0 || r >= G) return fail(SPARSP_ERR_INVALID, fn, "r must lie in [0, G)");
  int32_t n = 0;
  for (int32_t i = 0; i < nb; ++i) {
    if (placement[i] < 0 || placement[i] >= G) return fail(SPARSP_ERR_INVALID, fn, "placement value outside [0, G)");
    n += placement[i] == r;
  }
  *Lq = n;
  if (n > capacity || (n > 0 && !q_blocks)) return fail(SPARSP_ERR_INVALID, fn, "q_blocks capacity too small");
  int32_t k = 0;
  for (int32_t i = 0; i < nb; ++i)
    if (placement[i] == r) q_blocks[k++] = i;
  return SPARSP_OK;
}

int32_t sparsp_demand_union(const sparsp_geometry* geom, const uint8_t* mask, int64_t mask_pitch,
                            const int32_t* placement, uint64_t* demand, int32_t* seg_offsets, int32_t* slot_block,
                            int32_t* slot_head, int32_t* slot_of, void* stream) {
  static const char* fn = "sparsp_demand_union";
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if ((st = check_mask(d, mask, mask_pitch, fn))) return st;
  if (!placement || !demand || !seg_offsets || !slot_block || !slot_head || !slot_of)
    return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (sparsp::compact_lds_bytes(d) > (size_t)sparsp::kCompactLdsLimit)
    return fail(SPARSP_ERR_UNSUPPORTED, fn, "G*W*12 + (G*H+1)*4 exceeds 64 KiB of LDS");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = sparsp::launch_union(d, mask, mask_pitch, demand, s);
  if (e == hipSuccess) e = sparsp::launch_compact(d, placement, demand, seg_offsets, slot_block, slot_head, slot_of, s);
  return hip_status(e, fn);
}

int32_t sparsp_pack_kv(const sparsp_geometry* geom, const uint16_t* K, const uint16_t* V, const int32_t* seg_offsets,
                       const int32_t* slot_block, const int32_t* slot_head, int32_t slot_capacity, uint16_t* packed,
                       void* stream) {
  static const char* fn = "sparsp_pack_kv";
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if (!K || !V || !seg_offsets || !slot_block || !slot_head || !packed) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (slot_capacity < 1) return fail(SPARSP_ERR_INVALID, fn, "slot_capacity must be >= 1");
  if (!aligned16(K) || !aligned16(V) || !aligned16(packed))
    return fail(SPARSP_ERR_INVALID, fn, "K, V and packed must be 16-byte aligned");
  return hip_status(sparsp::launch_pack(d, K, V, seg_offsets, slot_block, slot_head, slot_capacity, packed,
                                        reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

namespace {

// Shared checks and launch of the attention entry points over the slot range [slot_lo, slot_hi) and the heads
// [h_lo, h_hi) (all heads when h_hi < 0); `anchored` for the single-pass call only.
int32_t attention_call(const char* fn, const sparsp_geometry* geom, const uint16_t* Q, const uint8_t* mask,
                       int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed, int32_t slot_lo,
                       int32_t slot_hi, float softmax_scale, float* O, float* lse, void* stream, int accumulate = 0,
                       int32_t h_lo = 0, int32_t h_hi = -1, int anchored = 0) {
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if (h_hi < 0) h_hi = d.H;
  if (h_lo < 0 || h_hi > d.H || h_lo > h_hi) return fail(SPARSP_ERR_INVALID, fn, "need 0 <= h_lo <= h_hi <= H");
  if ((st = check_mask(d, mask, mask_pitch, fn))) return st;
  if (d.Lq > 0 && (!Q || !slot_of || !packed || !O || !lse)) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(SPARSP_ERR_INVALID, fn, "softmax_scale must be finite and positive");
  if ((Q && !aligned16(Q)) || (packed && !aligned16(packed)) || (O && !aligned16(O)))
    return fail(SPARSP_ERR_INVALID, fn, "Q, packed and O must be 16-byte aligned");
  return hip_status(sparsp::launch_attention(d, Q, mask, mask_pitch, slot_of, packed, slot_lo, slot_hi, h_lo, h_hi,
                                             softmax_scale, O, lse, accumulate, anchored,
                                             reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

}  // namespace

int32_t sparsp_block_sparse_attn(const sparsp_geometry* geom, const uint16_t* Q, const uint8_t* mask,
                                 int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                 int32_t slot_capacity, float softmax_scale, float* O, float* lse, void* stream) {
  static const char* fn = "sparsp_block_sparse_attn";
  if (slot_capacity < 0) return fail(SPARSP_ERR_INVALID, fn, "slot_capacity must be >= 0");
  return attention_call(fn, geom, Q, mask, mask_pitch, slot_of, packed, 0, slot_capacity, softmax_scale, O, lse,
                        stream, 0, 0, -1, 1);
}

int32_t sparsp_block_sparse_attn_segment(const sparsp_geometry* geom, const uint16_t* Q, const uint8_t* mask,
                                         int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                         int32_t slot_lo, int32_t slot_hi, float softmax_scale, float* O, float* lse,
                                         void* stream) {
  static const char* fn = "sparsp_block_sparse_attn_segment";
  if (slot_lo < 0 || slot_hi < slot_lo) return fail(SPARSP_ERR_INVALID, fn, "need 0 <= slot_lo <= slot_hi");
  return attention_call(fn, geom, Q, mask, mask_pitch, slot_of, packed, slot_lo, slot_hi, softmax_scale, O, lse,
                        stream);
}

int32_t sparsp_block_sparse_attn_segment_accumulate(const sparsp_geometry* geom, const uint16_t* Q,
                                                    const uint8_t* mask, int64_t mask_pitch, const int32_t* slot_of,
                                                    const uint16_t* packed, int32_t slot_lo, int32_t slot_hi,
                                                    float softmax_scale, float* O, float* lse, void* stream) {
  static const char* fn = "sparsp_block_sparse_attn_segment_accumulate";
  if (slot_lo < 0 || slot_hi < slot_lo) return fail(SPARSP_ERR_INVALID, fn, "need 0 <= slot_lo <= slot_hi");
  return attention_call(fn, geom, Q, mask, mask_pitch, slot_of, packed, slot_lo, slot_hi, softmax_scale, O, lse,
                        stream, 1);
}

int32_t sparsp_block_sparse_attn_chunk_accumulate(const sparsp_geometry* geom, const uint16_t* Q, const uint8_t* mask,
                                                  int64_t mask_pitch, const int32_t* slot_of, const uint16_t* packed,
                                                  int32_t slot_lo, int32_t slot_hi, int32_t h_lo, int32_t h_hi,
                                                  float softmax_scale, float* O, float* lse, void* stream) {
  static const char* fn = "sparsp_block_sparse_attn_chunk_accumulate";
  if (slot_lo < 0 || slot_hi < slot_lo) return fail(SPARSP_ERR_INVALID, fn, "need 0 <= slot_lo <= slot_hi");
  if (h_lo < 0 || h_hi < h_lo) return fail(SPARSP_ERR_INVALID, fn, "need 0 <= h_lo <= h_hi <= H");
  return attention_call(fn, geom, Q, mask, mask_pitch, slot_of, packed, slot_lo, slot_hi, softmax_scale, O, lse,
                        stream, 1, h_lo, h_hi);
}

int32_t sparsp_chunk_plan(const int32_t* seg_offsets, const int32_t* counts, const int32_t* placement, int32_t G,
                          int32_t H, int32_t nb, int32_t r, int32_t chunks_steady, int32_t chunks_drain,
                          sparsp_chunk* chunks, int32_t capacity, int32_t* n_chunks) {
  static const char* fn = "sparsp_chunk_plan";
  if (!seg_offsets || !counts || !placement || !n_chunks) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (G < 1 || G > sparsp::kMaxRanks || H < 1 || nb < 1) return fail(SPARSP_ERR_INVALID, fn, "bad G, H or nb");
  if (r < 0 || r >= G) return fail(SPARSP_ERR_INVALID, fn, "r must lie in [0, G)");
  if (chunks_steady < 1 || chunks_drain < 1) return fail(SPARSP_ERR_INVALID, fn, "chunk counts must be >= 1");
  for (int32_t j = 0; j < nb; ++j)
    if (placement[j] < 0 || placement[j] >= G) return fail(SPARSP_ERR_INVALID, fn, "placement value outside [0, G)");
  for (int32_t i = 0; i < G * H; ++i)
    if (seg_offsets[i + 1] < seg_offsets[i] || seg_offsets[i] < 0)
      return fail(SPARSP_ERR_INVALID, fn, "seg_offsets must be a non-decreasing prefix from >= 0");
  // Selected tiles per (source rank, head): the access counts summed over the blocks each rank owns.
  std::vector<int64_t> tiles((size_t)G * H, 0);
  for (int32_t h = 0; h < H; ++h)
    for (int32_t j = 0; j < nb; ++j) tiles[(size_t)placement[j] * H + h] += counts[(size_t)h * nb + j];
  std::vector<sparsp_chunk> plan;
  for (int32_t k = 0; k < G; ++k) {
    const int32_t p = (r + k) % G;
    // The local segment stays whole; the final remote segment uses the drain count, the others the steady count.
    int32_t c = k == 0 ? 1 : (k == G - 1 ? chunks_drain : chunks_steady);
    if (c > H) c = H;
    const size_t first = plan.size();
    for (int32_t i = 0; i < c; ++i) {
      sparsp_chunk ch;
      ch.p = p;
      ch.h_lo = (int32_t)((int64_t)i * H / c);
      ch.h_hi = (int32_t)((int64_t)(i + 1) * H / c);
      ch.slot_lo = seg_offsets[p * H + ch.h_lo];
      ch.slot_hi = seg_offsets[p * H + ch.h_hi];
      ch.reserved = 0;
      ch.tiles = 0;
      for (int32_t h = ch.h_lo; h < ch.h_hi; ++h) ch.tiles += tiles[(size_t)p * H + h];
      if (ch.slot_hi > ch.slot_lo) plan.push_back(ch);
    }
    // Within the segment: most tiles first, so its chunk with the highest sparsity runs last (ties: lower
    // heads first: a stable insertion sort).
    for (size_t a = first + 1; a < plan.size(); ++a)
      for (size_t b = a; b > first && plan[b - 1].tiles < plan[b].tiles; --b) std::swap(plan[b - 1], plan[b]);
  }
  *n_chunks = (int32_t)plan.size();
  if ((int32_t)plan.size() > capacity || (!plan.empty() && !chunks))
    return fail(SPARSP_ERR_INVALID, fn, "chunk capacity too small");
  for (size_t i = 0; i < plan.size(); ++i) chunks[i] = plan[i];
  return SPARSP_OK;
}

int32_t sparsp_merge_partial(const sparsp_geometry* geom, float* O, float* lse, const float* O_part,
                             const float* lse_part, void* stream) {
  static const char* fn = "sparsp_merge_partial";
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if (d.Lq > 0 && (!O || !lse || !O_part || !lse_part)) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if ((O && !aligned16(O)) || (O_part && !aligned16(O_part)))
    return fail(SPARSP_ERR_INVALID, fn, "O and O_part must be 16-byte aligned");
  const int64_t rows = (int64_t)d.H * d.Lq * d.b;
  return hip_status(sparsp::launch_merge(rows, d.d, O, lse, O_part, lse_part, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

int32_t sparsp_placement_permutation(const int32_t* placement, int32_t nb, int32_t G, int32_t* pos,
                                     int32_t* rank_offsets) {
  static const char* fn = "sparsp_placement_permutation";
  if (!placement || !pos || !rank_offsets) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (nb < 1 || G < 1) return fail(SPARSP_ERR_INVALID, fn, "nb and G must be >= 1");
  for (int32_t j = 0; j < nb; ++j)
    if (placement[j] < 0 || placement[j] >= G) return fail(SPARSP_ERR_INVALID, fn, "placement value outside [0, G)");
  // Counting sort by rank: offsets are the exclusive prefix sums of the per-rank block counts, and a
  // running cursor per rank keeps ascending logical order inside a rank.
  std::vector<int32_t> cursor(G + 1, 0);
  for (int32_t j = 0; j < nb; ++j) ++cursor[placement[j] + 1];
  for (int32_t p = 0; p < G; ++p) cursor[p + 1] += cursor[p];
  for (int32_t p = 0; p <= G; ++p) rank_offsets[p] = cursor[p];
  for (int32_t j = 0; j < nb; ++j) pos[j] = cursor[placement[j]]++;
  return SPARSP_OK;
}

int32_t sparsp_permute_blocks(const void* src, void* dst, int64_t outer, int32_t nb, int64_t block_bytes,
                              const int32_t* pos, int32_t inverse, void* stream) {
  static const char* fn = "sparsp_permute_blocks";
  if (outer < 0) return fail(SPARSP_ERR_INVALID, fn, "outer must be >= 0");
  if (nb < 1) return fail(SPARSP_ERR_INVALID, fn, "nb must be >= 1");
  if (block_bytes < 16 || block_bytes % 16 != 0)
    return fail(SPARSP_ERR_INVALID, fn, "block_bytes must be a positive multiple of 16");
  if (outer == 0) return SPARSP_OK;
  if (!src || !dst || !pos) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (!aligned16(src) || !aligned16(dst)) return fail(SPARSP_ERR_INVALID, fn, "src and dst must be 16-byte aligned");
  if (src == dst) return fail(SPARSP_ERR_INVALID, fn, "src and dst must not overlap");
  if (outer > (int64_t)0x7fffffff / nb) return fail(SPARSP_ERR_UNSUPPORTED, fn, "outer*nb must be < 2^31");
  const hipError_t e = sparsp::launch_permute(src, dst, outer, nb, block_bytes, pos, inverse ? 1 : 0,
                                              reinterpret_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidConfiguration) return fail(SPARSP_ERR_UNSUPPORTED, fn, "grid exceeds 2^31 - 1 workgroups");
  return hip_status(e, fn);
}

int32_t sparsp_demand_counts(const sparsp_geometry* geom, const uint8_t* mask, int64_t mask_pitch, int32_t* counts,
                             void* stream) {
  static const char* fn = "sparsp_demand_counts";
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if ((st = check_mask(d, mask, mask_pitch, fn))) return st;
  if (!counts) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  return hip_status(sparsp::launch_counts(d, mask, mask_pitch, counts, reinterpret_cast<hipStream_t>(stream)), fn);
}

int32_t sparsp_comm_volume(const uint64_t* demand, int32_t G, int32_t H, int32_t nb, const int32_t* placement,
                           int64_t* direct, int64_t* relay, int64_t* dense) {
  static const char* fn = "sparsp_comm_volume";
  if (!demand || !placement || !direct || !relay || !dense) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (G < 1 || G > sparsp::kMaxRanks) return fail(SPARSP_ERR_INVALID, fn, "G must lie in [1, 64]");
  if (H < 1 || nb < 1) return fail(SPARSP_ERR_INVALID, fn, "H and nb must be >= 1");
  for (int32_t j = 0; j < nb; ++j)
    if (placement[j] < 0 || placement[j] >= G) return fail(SPARSP_ERR_INVALID, fn, "placement value outside [0, G)");
  const int64_t W = (nb + 63) / 64;
  std::vector<int64_t> dir((size_t)G * G, 0), rel((size_t)G * G, 0), den(G, 0);
  for (int32_t j = 0; j < nb; ++j) den[placement[j]] += (int64_t)(G - 1) * H;
  for (int32_t h = 0; h < H; ++h)
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t p = placement[j];
      int32_t far = 0;  // ring distance of the farthest consumer of (h, j)
      for (int32_t c = 0; c < G; ++c) {
        if (c == p) continue;
        const uint64_t word = demand[((int64_t)c * H + h) * W + j / 64];
        if ((word >> (j % 64)) & 1u) {
          ++dir[(size_t)c * G + p];
          const int32_t dist = (c - p + G) % G;
          if (dist > far) far = dist;
        }
      }
      for (int32_t k = 1; k <= far; ++k) ++rel[(size_t)p * G + k];
    }
  memcpy(direct, dir.data(), dir.size() * sizeof(int64_t));
  memcpy(relay, rel.data(), rel.size() * sizeof(int64_t));
  memcpy(dense, den.data(), den.size() * sizeof(int64_t));
  return SPARSP_OK;
}

int32_t sparsp_pool_blocks(const sparsp_geometry* geom, const uint16_t* X, int32_t n_blocks, const int32_t* block_ids,
                           float* pooled, void* stream) {
  static const char* fn = "sparsp_pool_blocks";
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if (n_blocks < 0 || n_blocks > d.nb) return fail(SPARSP_ERR_INVALID, fn, "n_blocks must lie in [0, nb]");
  if (d.H > 65535) return fail(SPARSP_ERR_UNSUPPORTED, fn, "H must be <= 65535");
  if (n_blocks == 0) return SPARSP_OK;
  if (!X || !pooled) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (!aligned16(X) || !aligned16(pooled)) return fail(SPARSP_ERR_INVALID, fn, "X and pooled must be 16-byte aligned");
  return hip_status(sparsp::launch_pool(d, X, n_blocks, block_ids, pooled, reinterpret_cast<hipStream_t>(stream)), fn);
}

int32_t sparsp_materialize_mask(const sparsp_geometry* geom, const float* q_pooled, const float* k_pooled,
                                float softmax_scale, float tau, int32_t k_min, uint8_t* mask, int64_t mask_pitch,
                                void* stream) {
  static const char* fn = "sparsp_materialize_mask";
  sparsp::Dims d;
  int32_t st = check_geometry(geom, fn, &d);
  if (st) return st;
  if ((st = check_mask(d, mask, mask_pitch, fn))) return st;
  if (d.nb > sparsp::kMaxSelectBlocks) return fail(SPARSP_ERR_UNSUPPORTED, fn, "nb must be <= 16384");
  if (d.H > 65535) return fail(SPARSP_ERR_UNSUPPORTED, fn, "H must be <= 65535");
  if (!(tau >= 0.f && tau <= 1.f)) return fail(SPARSP_ERR_INVALID, fn, "tau must lie in [0, 1]");
  if (k_min < 0) return fail(SPARSP_ERR_INVALID, fn, "k_min must be >= 0");
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(SPARSP_ERR_INVALID, fn, "softmax_scale must be finite and positive");
  if (d.Lq == 0) return SPARSP_OK;
  if (!q_pooled || !k_pooled) return fail(SPARSP_ERR_INVALID, fn, "NULL pointer");
  if (!aligned16(q_pooled) || !aligned16(k_pooled))
    return fail(SPARSP_ERR_INVALID, fn, "q_pooled and k_pooled must be 16-byte aligned");
  return hip_status(sparsp::launch_select(d, q_pooled, k_pooled, softmax_scale, tau, k_min, mask, mask_pitch,
                                          reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
