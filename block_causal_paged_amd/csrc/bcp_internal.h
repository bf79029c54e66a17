// Internal definitions shared by the host ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bcp.h"

namespace bcp {

// Attention tiling. One workgroup owns 256 packed query rows: tile_q consecutive live
// positions of one sequence times the G = Hq/Hkv query heads that share one kv head,
// packed position-major (row rho = position * G + head-in-group). Keys stream in tiles of
// kTileK rows.
constexpr int kTileK = 64;
constexpr int kRowsPerWG = 256;
constexpr int kNarrowRows = 64;   // packed rows of a narrow work item (short live blocks)
constexpr int kMaxBandKeyTiles = 2048;   // key tiles per q-tile row with a window in mode B

// Split-KV planning. The work of a step is the sequence of (kv head, unit, key tile)
// visits, ordered by kv head, then unit, then tile (a unit is one (sequence, q-tile); its
// key tiles are the non-skipped ones). It is cut into at most kWGs near-equal contiguous
// ranges, each at least kMinChunk visits long when the step has that much work. Range r
// runs on workgroup (r % kPerXcd) * kXcds + r / kPerXcd: workgroups are dealt to the XCDs
// in turn, so each XCD gets kPerXcd consecutive ranges, mostly of one kv head, whose keys
// and values then stay in that XCD's L2 across the q-tiles that reuse them.
// A range holds whole (unit, head) pairs plus at most one piece at each end; a pair cut by
// range boundaries is computed in pieces, each writing a normalized partial result that
// the combine kernel merges. There are fewer than kWGs boundaries and each lies inside at
// most one pair, so fewer than kWGs pairs are split and they have fewer than 2*kWGs pieces.
constexpr int kWGs = 256;
constexpr int kXcds = 8;
constexpr int kPerXcd = kWGs / kXcds;
constexpr int kMinChunk = 4;
constexpr int kMaxPartialSlots = 2 * kWGs;

constexpr int kNegInfBlk = INT32_MIN;   // a committed row in mode A: seen by every live row
constexpr int kNoKeyBlk = INT32_MAX;    // an absent key: seen by nobody

// Step plan, in int32 words:
//   [0, 16)                 header (kHdr* below): n_items, n_split, workgroups used, total
//                           tiles T, tile_q, tile_k, nqt, nkt, a magic word, batch, Hkv, a
//                           hash of every sequence's live rows and committed length, the
//                           window, mode B, total_q, the per-sequence capacity
//                           max_pages_per_seq * page_size -- the attention and combine kernels
//                           do nothing unless the shape words match their own arguments (every
//                           item field the planner wrote then lies inside this call's
//                           buffers), and checked mode compares the whole header with the meta
//   rng   [kWGs][12]        per range: first item, end item, a copy of the first item's 8
//                           words (when the range is not empty), 0, 0 -- so a workgroup
//                           starts from one load; right after the header, at a place that
//                           does not depend on the step's shape, so that a workgroup loads its
//                           record together with the header and checks both at once
//   split [kWGs][4]         unit, kv head, first partial slot, number of pieces (also at a
//                           fixed place, for the combine kernel)
//   cnt   [U]               non-skipped key tiles per unit (U = batch * nqt)
//   list  [U * nkt]         per unit, its non-skipped virtual tile indices in order, each
//                           stored as (t << 1) | is_partial; t < nct is cached tile t,
//                           t >= nct is live tile t - nct
//   upre  [U + 1]           exclusive prefix sums of cnt (upre[U] = T)
//   wg    [kWGs + 1]        first item of each range; wg[kWGs] = n_items
//   items [max_items][8]    unit, kv head, first ordinal, end ordinal, partial slot (-1 when
//                           the item is a whole pair), and the unit's sequence's first live
//                           row, live-row count and committed length (clamped to the pages)
constexpr int kItemWords = 8;
constexpr int kRngWords = 12;
constexpr int kHdrWords = 16;
enum {
  kHdrItems = 0, kHdrSplit = 1, kHdrWgs = 2, kHdrTiles = 3, kHdrTileQ = 4, kHdrTileK = 5,
  kHdrNqt = 6, kHdrNkt = 7, kHdrMagic = 8, kHdrBatch = 9, kHdrHkv = 10, kHdrLenHash = 11,
  kHdrWindow = 12, kHdrModeB = 13, kHdrTotalQ = 14, kHdrKvCap = 15
};
constexpr int kPlanMagic = 0x32504342;   // "BCP2"

// Hash of one sequence's live rows (first row q0, count ql) and committed length kvl, as the
// planner clamps them; the plan header holds the wrapping sum over the sequences. It is
// MurmurHash3's 32-bit finalizer applied in a chain, so a stale plan (one built before a
// commit moved kv_len, say) is told apart from the current step in checked mode.
__host__ __device__ inline uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}
__host__ __device__ inline uint32_t seq_len_hash(int s, int q0, int ql, int kvl) {
  uint32_t x = fmix32((uint32_t)s * 0x9E3779B1u ^ (uint32_t)q0);
  x = fmix32(x ^ (uint32_t)ql * 0x27D4EB2Fu);
  return fmix32(x ^ (uint32_t)kvl * 0x165667B1u);
}

struct PlanLayout {
  int64_t cnt, list, upre, wg, items, split, rng, words;
  int units, nkt, max_items;
};

__host__ __device__ inline PlanLayout plan_layout(int batch, int nqt, int nkt, int hkv) {
  PlanLayout p;
  p.units = batch * nqt;
  p.nkt = nkt;
  p.max_items = p.units * hkv + kWGs;
  p.rng = kHdrWords;
  p.split = p.rng + kRngWords * (int64_t)kWGs;
  p.cnt = p.split + 4 * (int64_t)kWGs;
  p.list = p.cnt + p.units;
  p.upre = p.list + (int64_t)p.units * nkt;
  p.wg = p.upre + p.units + 1;
  p.items = p.wg + kWGs + 1;
  p.words = p.items + kItemWords * (int64_t)p.max_items;
  return p;
}

struct ClassifyArgs {
  const int32_t* cu_q;
  const int32_t* kv_len;
  const int32_t* page_table;
  const int32_t* q_blk;
  const int32_t* kv_blk;
  uint8_t* tile_class;    // may be null
  int32_t* phys_page;     // may be null
  int32_t* plan;          // may be null
  int batch, total_q, tile_q, tile_k, nqt, nct, nkt, block_size, page_size, num_pages,
      max_pages, max_q_len, mode_b, phys_per_tile, phys_tiles, num_kv_heads;
  int grid_q;             // q-tile workgroups per sequence: max(nqt, 1)
  int window;             // sliding window in positions, 0 for none
  const int32_t* q_pos;   // mode B with a window: position of each live row
  const int32_t* kv_pos;  //   and of each cache slot
};

struct PlanArgs {
  int32_t* plan;
  const int32_t* cu_q;
  const int32_t* kv_len;
  int batch, nqt, nkt, num_kv_heads, tile_q, tile_k;
  int total_q, max_q_len, kv_cap;   // kv_cap = max_pages_per_seq * page_size
  int window, mode_b;               // recorded in the header (with total_q and kv_cap)
  // Small mode-A steps without a window: the planner classifies the tiles itself (closed form)
  // and writes the tile lists, and the classes and physical pages when asked, so that
  // build_tile_mask is one launch.
  int fused;
  int nct, block_size, page_size, num_pages, max_pages, phys_per_tile;
  uint8_t* tile_class;              // may be null
  int32_t* phys_page;               // may be null
  const int32_t* page_table;
};
// Largest class and page-entry count of a step the planner classifies itself.
constexpr int kFusedPlanElems = 4096;

struct AttnArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* k_cache;
  const void* v_cache;
  void* out;
  float* lse;
  float* part_o;          // [kMaxPartialSlots][256][d] normalized partial outputs (fp32 steps)
  uint16_t* part_h;       // the same in fp16 (bf16 steps), each row scaled by part_scale's inverse
  float* part_scale;      // [kMaxPartialSlots][256] factor that restores an fp16 partial row
  float* part_lse;        // [kMaxPartialSlots][256] log2-domain partial LSE (slot = piece)
  const int32_t* cu_q;
  const int32_t* kv_len;
  const int32_t* page_table;
  const int32_t* q_blk;
  const int32_t* kv_blk;
  const int32_t* plan;
  unsigned long long* stats;
  int batch, total_q, max_q_len, Hq, Hkv, G, tile_q, nqt, nkt, nct, page_size, num_pages,
      max_pages, block_size, mode_b, max_items;
  int page_shift;         // log2(page_size) when it is a power of two, else -1
  int window;             // sliding window in positions, 0 for none
  int live_in_cache;      // live row i of a sequence is read from the pool at kv_len + i
  const int32_t* q_pos;   // mode B with a window: position of each live row
  const int32_t* kv_pos;  //   and of each cache slot
  float scale_log2;       // softmax scale times log2(e)
};

struct CommitArgs {
  const void* k_src;
  const void* v_src;
  void* k_cache;
  void* v_cache;
  const int32_t* cu_src;
  const int32_t* src_row;
  const int32_t* dst_start;
  const int32_t* src_blk;
  int32_t* kv_blk_out;
  const int32_t* page_table;
  int batch, total, n_src, row_chunks, page_size, num_pages, max_pages;
};

hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream);
hipError_t launch_planner(const PlanArgs& a, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_attn_bf16_narrow(const AttnArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_combine(const AttnArgs& a, int head_dim, int is_bf16, int grid,
                          hipStream_t stream);
hipError_t launch_commit(const CommitArgs& a, int grid, hipStream_t stream);

// ----------------------------------------------------------------------------------------
// Range of the step plan that workgroup `wg` works through (see the split-KV planning).
__host__ __device__ inline int range_of_wg(int wg) { return (wg % kXcds) * kPerXcd + wg / kXcds; }

// Device helpers shared by the kernels.
// ----------------------------------------------------------------------------------------
#ifdef __HIPCC__
// Page translation: physical page of logical row j of sequence s, or -1 when the row lies
// beyond max_pages_per_seq pages or its page id is outside the pool ("Paged Attention":
// the page table maps logical rows onto physical pages).
__device__ __forceinline__ int translate_page(const int32_t* __restrict__ page_table, int s, int j,
                                              int page_size, int max_pages, int num_pages) {
  if (j < 0) return -1;
  int lp = j / page_size;
  if (lp >= max_pages) return -1;
  int p = page_table[(int64_t)s * max_pages + lp];
  return (p >= 0 && p < num_pages) ? p : -1;
}

// Row j's logical page and slot, with shifts when the page size is a power of two.
__device__ __forceinline__ void page_split(int j, int page_size, int page_shift, int* lp, int* slot) {
  if (page_shift >= 0) {
    *lp = j >> page_shift;
    *slot = j & (page_size - 1);
  } else {
    *lp = j / page_size;
    *slot = j - *lp * page_size;
  }
}

// Read-only device data through the scalar cache when the address is uniform.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ cint32* as_const(const int32_t* p) { return (cint32*)p; }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Live rows of sequence s, clamped so that [*q0, *q0 + *q_len) lies inside [0, total_q).
__device__ __forceinline__ void live_rows(const int32_t* __restrict__ cu_q, int s, int total_q,
                                          int max_q_len, int* q0, int* q_len) {
  const int a = clampi(cu_q[s], 0, total_q);
  *q0 = a;
  *q_len = clampi(cu_q[s + 1] - a, 0, min(max_q_len, total_q - a));
}

// True when the plan header describes the step these arguments describe (its shape words;
// the length hash is compared on the host in checked mode). Every kernel that reads a plan
// does nothing when it is false. When it is true, every field the planner wrote lies inside
// this call's buffers: units, kv heads, tile ordinals and partial slots by the shape, the
// live rows by total_q, the committed lengths by the per-sequence capacity.
// h: header words kHdrTileQ .. kHdrKvCap, already loaded (so that a caller can load them
// together with its range record).
struct PlanShape {
  int w[kHdrWords - kHdrTileQ];
};
__device__ __forceinline__ PlanShape plan_shape(cint32* plan) {
  PlanShape h;
#pragma unroll
  for (int i = 0; i < kHdrWords - kHdrTileQ; ++i) h.w[i] = plan[kHdrTileQ + i];
  return h;
}
__device__ __forceinline__ bool plan_matches(const PlanShape& h, const AttnArgs& a) {
  // Every comparison is evaluated (no short-circuit branches): one scalar AND chain.
  auto eq = [&](int k, int v) { return (int)(h.w[k - kHdrTileQ] == v); };
  return (eq(kHdrMagic, kPlanMagic) & eq(kHdrTileQ, a.tile_q) & eq(kHdrTileK, kTileK) & eq(kHdrNqt, a.nqt) &
          eq(kHdrNkt, a.nkt) & eq(kHdrBatch, a.batch) & eq(kHdrHkv, a.Hkv) & eq(kHdrWindow, a.window) &
          eq(kHdrModeB, a.mode_b) & eq(kHdrTotalQ, a.total_q) & eq(kHdrKvCap, a.max_pages * a.page_size)) != 0;
}
__device__ __forceinline__ bool plan_matches(cint32* plan, const AttnArgs& a) {
  return plan_matches(plan_shape(plan), a);
}

// One work item of the plan: (unit, kv head, first and end tile ordinal, partial slot or
// -1, the unit's sequence's first live row, live-row count and committed length).
struct PlanItem {
  int u, g, ob, oe, pslot, q0, q_len, kvl;
};
__device__ __forceinline__ void read_item(cint32* ip, PlanItem* it) {
  it->u = ip[0];
  it->g = ip[1];
  it->ob = ip[2];
  it->oe = ip[3];
  it->pslot = ip[4];
  it->q0 = ip[5];
  it->q_len = ip[6];
  it->kvl = ip[7];
}
#endif

}  // namespace bcp
