// Block-causal paged attention for bf16 inputs on gfx950 matrix cores.
//
// What is computed ("Inference for Interpretable Text-Diffusion Models", Background and
// "FlexAttention with Aligned Tiles"; "Inference: Fewer, smaller forwards", Advancement 1):
// every live row attends to the committed rows of its sequence (gathered through the page
// table, section "Paged Attention") and to the live rows of its own and earlier blocks,
// with a numerically stable online softmax (running max and sum, rescaling the output
// whenever the max grows). Tiles the step plan marks as skipped are never loaded; only
// partial tiles evaluate the mask.
//
// Work decomposition. A workgroup of 8 waves works through the items of its range of the
// step plan; an item is one kv head g, one q-tile of a sequence (tile_q positions x the G
// query heads of g = 256 packed rows, rho = position * G + head), and a contiguous run of
// that q-tile's non-skipped key tiles. Wave w owns packed rows [32w, 32w+32), one
// 32-column MFMA block. Waves 0-3 and 4-7 form two groups with one wave of each on every
// SIMD; barriers cut time into half-steps and the second group runs half a step behind
// the first, so one wave's matrix instructions overlap the other's softmax.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, wave64). Scores are computed
// transposed, S^T = K Q^T: K rows are the A operand, queries the B operand (held in
// registers for the whole item), so each lane owns one query column and 16 key rows of
// every 32x32 block. The row max and row sum of the softmax are in-lane reductions plus
// one exchange with lane^32. The output is also accumulated transposed, O^T += V^T P^T,
// with P^T taken straight from the score registers: the 8 keys a lane half contributes to
// one PV step are exactly the 8 score values it already holds, which fixes a permutation
// of the keys inside every 16-key group. V stays row-major in LDS; gfx950's LDS transpose
// read (ds_read_b64_tr_b16) hands each lane 4 keys of one d column, and two of them per
// step deliver exactly those 8 keys as the A operand.
//
// Staging. Key and value tiles move HBM -> LDS with direct loads (global_load_lds_dwordx4),
// without passing through registers, into a 3-stage key ring and a 4-stage value ring;
// each group issues its loads two (first group) or three (second group) tiles ahead. The
// plan's tile lists and, per (tile, wave), the first memory row of the wave's 8 rows are
// staged in LDS a window of 256 tiles at a time, so the tile loop issues no memory loads
// other than the tiles' own. When the page size is a multiple of 8 a wave's 8 rows are one
// run in memory (one scalar base plus fixed per-lane offsets); when they are not (smaller
// pages, a run cut by the end of the committed or live rows, an invalid page) the window
// holds -1 and the wave resolves each row itself; absent rows load the sequence's first
// live row in their place, and the mask gives them no weight.
#include "bcp_internal.h"

#include <type_traits>

namespace bcp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKStages = 3;                     // key tile ring
constexpr int kVStages = 4;                     // value tile (and key block id) ring
constexpr int kRowsPerWave = kTileK / kWaves;   // key rows each wave stages per tile

// LDS: key and value tiles are row-major [64 keys][d] with no padding, so one direct-load
// wave instruction (a contiguous 1 KB run) fills whole rows; the 16-byte chunks of each
// row are XOR-swizzled (kswz, vswz) so that the operand reads hit distinct banks.
// The item's plan entries are staged in LDS one window of kWin tiles at a time, with, for
// each tile and wave, the memory row of the wave's first key row when all 8 of its rows are
// present and consecutive in memory (-1 otherwise). Each wave owns a 4 KB output staging
// area (32 rows x 128 bytes), through which the epilogue turns its column-held results into
// whole 128-byte row segments before storing them.
constexpr int kWin = 256;
constexpr int kWinPerThread = kWin * kWaves / kThreads;   // window slots each thread stages
constexpr int kEpRowBytes = 128;
constexpr int kLivePages = 256;   // pages of an item's live rows staged in LDS when those sit in the pool
template <int HD>
struct AttnSmem {
  uint16_t k[kKStages][kTileK * HD];
  uint16_t v[kVStages][kTileK * HD];
  int kblk[kVStages][kTileK];      // block id of each key of a partial tile
  int kpos[kVStages][kTileK];      // and its position (mode B with a window)
  int win_e[kWin];                 // the item's plan entries, one window at a time
  int win_row[kWin][kWaves];       // first memory row of each wave's 8 rows, or -1
  int live_pg[kLivePages];         // physical pages of the live rows' logical pages, when in the pool
  float ep[kWaves][32 * kEpRowBytes / 4];   // per-wave output staging
};

// K operand reads: 16 lanes read rows r..r+15 at one logical chunk, so the swizzle spreads
// consecutive rows over all 16-byte bank groups. V transpose reads: 32 lanes read 4
// consecutive rows x 8 bytes x 8, so the swizzle moves each of the 4 rows to its own
// 64-byte window.
template <int HD>
__device__ __forceinline__ int kswz(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int HD>
__device__ __forceinline__ int vswz(int r) { return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Direct global->LDS copies, written as inline assembly so the compiler does not attach
// its conservative wait before every LDS read (it cannot tell the stage being filled from
// the one being read); the kernel waits for them itself. Lane i of the wave writes LDS
// bytes [lds + size*i, +size). `lds` is wave-uniform at every call. The key and value
// loads carry the non-temporal hint (nt): each tile is streamed through the cache once per
// work item, and measured, the hint shortens the decode steps by a fifth to a third.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ unsigned uni(unsigned x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const void* uni(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  return (const void*)(uintptr_t)((uint64_t)uni((unsigned)x) | ((uint64_t)uni((unsigned)(x >> 32)) << 32));
}
// Per-lane 64-bit address.
__device__ __forceinline__ void dma16(const void* g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(uni(lds)), "v"(g) : "memory");
}
// Wave-uniform base plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16s(const void* base, unsigned off, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(uni(lds)), "v"(off), "s"(uni(base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(uni(lds)), "v"(g) : "memory");
}
// Wait until at most n of this wave's vector-memory loads are outstanding (they complete
// in issue order, so everything issued before the last n has landed). n is 0 or a tile's
// loads: 2*NI, plus one or two for partial mode-B tiles, NI being 1 or 2.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
  }
}

// Scheduling pattern for the matrix phase: after AHEAD LDS reads, each of the NM matrix
// instructions is followed by its share of the remaining NR - AHEAD reads.
template <int NM, int NR, int AHEAD, int I = 0>
__device__ __forceinline__ void interleave() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int lo = AHEAD + (I * (NR - AHEAD)) / NM, hi = AHEAD + ((I + 1) * (NR - AHEAD)) / NM;
    if constexpr (hi > lo) __builtin_amdgcn_sched_group_barrier(0x100, hi - lo, 0);
    interleave<NM, NR, AHEAD, I + 1>();
  }
}

// max(x[l % 32], x[l % 32 + 32]) in every lane l: the max over the two halves of the wave,
// exchanged with a cross-half lane swap instead of an LDS round trip.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }

// The same exchange for a sum: x[l % 32] + x[l % 32 + 32].
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A split piece's partial output is stored in fp16, each row multiplied by a power of two
// that puts its largest magnitude in [2^13, 2^14): fp16 then keeps 11 significant bits of
// every value of the row that matters and cannot overflow, whatever the values' scale. amax
// is the largest |O| of this lane's half of the row before the division by the row sum,
// inv that division; returns the factor for this lane's values and sets *restore to what
// the merge multiplies the stored row by.
__device__ __forceinline__ float piece_factor(float amax, float inv, float* restore) {
  const int e = clampi(__builtin_amdgcn_frexp_expf(half_max(amax) * inv), -100, 126);
  *restore = __builtin_amdgcn_ldexpf(1.f, e - 14);
  return __builtin_amdgcn_ldexpf(inv, 14 - e);
}

// P = 2^(s * sl2 - m) of one 64-key tile for this lane's 32 scores, in bf16 for the PV
// product; returns the lane's sum of the fp32 values (a tree per 8 keys).
__device__ __forceinline__ float tile_exp(const f32x16 (&sc)[2], float sl2, float m, bf16x8 (&pf)[2][2]) {
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      f32x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * hs + e], sl2, -m));
      pf[kb][hs] = to_bf16x8(x);
      rs += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
    }
  return rs;
}

// Online softmax of one tile (log2 domain), for the query row this lane holds half of.
// The reference m is lazy: it starts at 0 and moves only when needed, and numerator (O)
// and denominator (l) both use it, so the result is the softmax whatever its value. The
// tile's P is first taken against the current m, and the row sum doubles as the check:
// only when some lane's sum exceeds 2^16 (a value may have outgrown the reference) or a
// row with no mass yet gets a sum below 2^-64 (its values may vanish) does the wave take
// the row max (over both lane halves) and, where it is more than 2^8 above m or is the
// row's first visible key, move m to it, rescale O and l, and take P again. So P <= 2^16
// always (bf16 and the fp32 sums hold it with room to spare), and no per-tile max is
// needed while the scores stay in range.
constexpr float kSumHi = 65536.f, kSumLo = 0x1p-64f;
template <int NDB>
__device__ __forceinline__ void tile_softmax(const f32x16 (&sc)[2], float sl2, float& m, float& l, f32x16 (&o)[NDB],
                                             bf16x8 (&pf)[2][2]) {
  float rs = tile_exp(sc, sl2, m, pf);
  const bool redo = !(rs <= kSumHi) || (l == 0.f && rs < kSumLo);
  if (__builtin_amdgcn_ballot_w64(redo)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][v]);
    const float mcand = half_max(mx) * sl2;   // -inf when no key of the tile is visible
    const bool first = half_sum(l) == 0.f;    // no mass yet: O and l are 0
    const bool grow = mcand > m + 8.f || (first && mcand != -INFINITY);
    const float alpha = grow && !first ? __builtin_amdgcn_exp2f(m - mcand) : 1.f;
    m = grow ? mcand : m;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    rs = tile_exp(sc, sl2, m, pf);
  }
  l += rs;
}

struct Item {
  int s, g, q0, q_len, kvl;
  int lp_live;   // logical page of row kv_len (the first live row when they sit in the pool)
};

template <int HD>
struct DmaShape {
  static constexpr int CPR = HD / 8;                    // 16-byte chunks per row
  static constexpr int RPI = 1024 / (2 * HD);           // rows per 1 KB wave instruction
  static constexpr int NI = kRowsPerWave / RPI;         // instructions per wave per matrix
};

// Number of keys of tile vt that exist (the rest of a partial tile is masked).
__device__ __forceinline__ int tile_valid(const AttnArgs& a, const Item& it, int vt) {
  return vt < a.nct ? clampi(it.kvl - vt * kTileK, 0, kTileK) : clampi(it.q_len - (vt - a.nct) * kTileK, 0, kTileK);
}

// Plan entry of a unit's o-th non-skipped key tile in mode A without a window, from the
// unit's lengths alone (the same entry the planner writes): the non-skipped tiles are the
// first nc cached tiles, then the first live tiles; a cached tile is partial only where the
// committed rows end inside it, a live tile unless all its keys exist and lie in blocks no
// later than the q-tile's first row's (qmin).
__device__ __forceinline__ int mode_a_entry(const AttnArgs& a, const Item& it, int nc, int qmin, int o) {
  if (o < nc) return (o << 1) | (it.kvl - o * kTileK < kTileK ? 1 : 0);
  const int lo = (o - nc) * kTileK, nv = min(it.q_len - lo, kTileK);
  return ((a.nct + o - nc) << 1) | (nv == kTileK && (lo + nv - 1) / a.block_size <= qmin ? 0 : 1);
}
__device__ __forceinline__ int mode_a_cached(const AttnArgs& a, const Item& it) {
  return min((it.kvl + kTileK - 1) / kTileK, a.nct);
}

// Staging state of one key tile for one wave: the plan entry and the memory row of the
// wave's first key row (rows of the kv cache for a cached tile, and for a live tile when
// the live rows are read from the pool; else rows of the new keys), -1 when the wave's
// rows need the general path, -(row) - 2 for a run of live rows in the pool that crosses
// into the next page (row: its first row).
struct Stage {
  int e;              // plan entry: (tile << 1) | is_partial; -1 when there is no tile
  int row0;
};

// Tile metadata as read from LDS for window position wi. Reading only issues the LDS loads
// (at a clamped, always valid position, so that no value has to be merged before it
// arrives); they are used one phase later, so the loop never waits for them.
struct RawMeta {
  int e, row0;
  bool valid;       // wi < nt
};

template <class Smem>
__device__ __forceinline__ RawMeta meta_read(int wi, int nt, int q, const Smem& sm) {
  const int w = min(wi, kWin - 1);
  RawMeta r;
  r.valid = wi < nt;
  r.e = sm.win_e[w];
  r.row0 = sm.win_row[w][q];
  return r;
}

// Make the entry and the row wave-uniform (they are the same in every lane).
__device__ __forceinline__ Stage meta_resolve(const RawMeta& r) {
  Stage st;
  st.e = r.valid ? uni(r.e) : -1;
  st.row0 = uni(r.row0);
  return st;
}

// Per-lane byte offsets of the fast staging path: row k*RPI + lane/CPR of the wave's 8-row
// run, at the swizzled chunk, relative to the run's first row.
template <int HD>
struct FastOffsets {
  unsigned k[DmaShape<HD>::NI], v[DmaShape<HD>::NI];
};

// Issue the direct loads of 8-row run q (rows 8q..8q+7) of a resolved tile into key stage
// `sk` and value stage `sv` (whose LDS byte addresses are klds and vlds): NI K and NI V wave instructions, plus one block-id copy for
// partial mode-B tiles. Returns the number of loads issued. When the run's 8 rows are
// present and consecutive in memory (row0 >= 0), one wave-uniform base and fixed per-lane
// offsets (fo, made for a run of the same parity) address them. Otherwise each lane
// resolves its own row through the page table, and a key past its region's length copies
// the sequence's first live row (its first query row when the live rows are read from the
// pool): such keys only occur in partial tiles, where the mask gives them weight exactly 0,
// and that row is finite, so they add exactly nothing. A key whose page id lies outside the
// pool (invalid metadata, which checked mode rejects) is loaded from that same row so that
// no load leaves the buffers; it keeps its place in the softmax, so the result for such
// input is unspecified.
template <int HD, int NI, bool BAND_B, class Smem>
__device__ __forceinline__ int stage_fetch(const AttnArgs& a, const Item& it, const Stage st, Smem& sm,
                                           int sk, int sv, unsigned klds, unsigned vlds,
                                           const FastOffsets<HD>& fo, int q) {
  using D = DmaShape<HD>;
  if (st.e < 0) return 0;
  const int vt = st.e >> 1;
  const int lane = threadIdx.x & 63;
  const bool cached = vt < a.nct;
  const bool paged = cached || a.live_in_cache;   // the tile's rows sit in the cache pool
  const uint16_t* kb = (const uint16_t*)(paged ? a.k_cache : a.k_new);
  const uint16_t* vb = (const uint16_t*)(paged ? a.v_cache : a.v_new);
  const int run0 = kRowsPerWave * q;              // first tile row of the run
  if (st.row0 >= 0) {
    const int64_t e0 = ((int64_t)st.row0 * a.Hkv + it.g) * HD;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int base = (run0 + k * D::RPI) * HD;
      dma16s(kb + e0, fo.k[k], klds + 2u * base);
      dma16s(vb + e0, fo.v[k], vlds + 2u * base);
    }
  } else if (st.row0 <= -2) {
    // Live rows in the pool whose run crosses a page boundary: the first `split` rows from
    // the run's page, the rest from the next one (its id staged in LDS with the item).
    const int row0 = -st.row0 - 2;
    int lp0, slot0;
    page_split(it.kvl + (vt - a.nct) * kTileK + run0, a.page_size, a.page_shift, &lp0, &slot0);
    const int split = a.page_size - slot0;
    const int64_t row1 = (int64_t)uni(sm.live_pg[lp0 + 1 - it.lp_live]) * a.page_size - split;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int rr = k * D::RPI + lane / D::CPR, r = run0 + rr, pch = lane % D::CPR;
      const int64_t row = rr < split ? row0 + rr : row1 + rr;
      const int base = (run0 + k * D::RPI) * HD;
      dma16(kb + (row * a.Hkv + it.g) * HD + 8 * (pch ^ kswz<HD>(r)), klds + 2u * base);
      dma16(vb + (row * a.Hkv + it.g) * HD + 8 * (pch ^ vswz<HD>(r)), vlds + 2u * base);
    }
  } else {
    const int nvalid = tile_valid(a, it, vt);
    const int32_t* pt = a.page_table + (int64_t)it.s * a.max_pages;
    // Substitute row for absent keys: the item's first live key row, or, when the live
    // rows are read from the pool, the item's first query row (equally finite).
    const uint16_t* ksub = (const uint16_t*)a.k_new + ((int64_t)it.q0 * a.Hkv + it.g) * HD;
    const uint16_t* vsub = (const uint16_t*)a.v_new + ((int64_t)it.q0 * a.Hkv + it.g) * HD;
    if (a.live_in_cache)
      ksub = vsub = (const uint16_t*)a.q + ((int64_t)it.q0 * a.Hq + (int64_t)it.g * a.G) * HD;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r = run0 + k * D::RPI + lane / D::CPR;   // row inside the tile
      const int pch = lane % D::CPR;                     // physical chunk
      int64_t row = -1;
      if (r < nvalid) {
        if (paged) {
          // Logical cache row: committed row j, or live row i at kv_len + i. A live row's
          // page comes from LDS (staged with the item) when it is among the first
          // kLivePages of the live region, so no load in the tile loop waits on memory.
          const int j = cached ? vt * kTileK + r : it.kvl + (vt - a.nct) * kTileK + r;
          int lp, slot;
          page_split(j, a.page_size, a.page_shift, &lp, &slot);
          int p;
          if (!cached && lp - it.lp_live < kLivePages) p = sm.live_pg[lp - it.lp_live];
          else p = pt[min(lp, a.max_pages - 1)];
          if (p >= 0 && p < a.num_pages) row = (int64_t)p * a.page_size + slot;
        } else {
          row = it.q0 + (vt - a.nct) * kTileK + r;
        }
      }
      const bool ok = row >= 0;
      const uint16_t* ksrc = ok ? kb + (row * a.Hkv + it.g) * HD : ksub;
      const uint16_t* vsrc = ok ? vb + (row * a.Hkv + it.g) * HD : vsub;
      const int base = (run0 + k * D::RPI) * HD;
      dma16(ksrc + 8 * (pch ^ kswz<HD>(r)), klds + 2u * base);
      dma16(vsrc + 8 * (pch ^ vswz<HD>(r)), vlds + 2u * base);
    }
  }
  // Block ids of a partial tile's keys: each wave handles its own 8 rows (lanes 0..7).
  // Mode A needs no memory; mode B copies them with an exec-masked 4-byte direct load
  // (inactive lanes issue no request).
  if (st.e & 1) {
    const int nvalid = tile_valid(a, it, vt);
    const int r = run0 + (lane & 7);
    const int j = (cached ? vt : vt - a.nct) * kTileK + r;
    if (!a.mode_b) {
      if (lane < 8) sm.kblk[sv][r] = r >= nvalid ? kNoKeyBlk : (cached ? kNegInfBlk : j / a.block_size);
    } else {
      // Keys that exist take their id from memory; absent keys get the id nobody sees. A
      // key in a page outside the pool (invalid metadata; its K and V were replaced by the
      // sequence's first live row) reads that row's id instead, so no load leaves the
      // buffers; the result for such input is unspecified.
      if constexpr (!BAND_B) {
        const int32_t* src = a.q_blk + it.q0;
        if (r < nvalid) {
          if (!cached) {
            src = a.q_blk + it.q0 + j;
          } else if (st.row0 >= 0) {
            src = a.kv_blk + st.row0 + (lane & 7);
          } else {
            int lp, slot;
            page_split(j, a.page_size, a.page_shift, &lp, &slot);
            const int p = a.page_table[(int64_t)it.s * a.max_pages + min(lp, a.max_pages - 1)];
            if (p >= 0 && p < a.num_pages) src = a.kv_blk + (int64_t)p * a.page_size + slot;
          }
        }
        if (lane < 8 && r >= nvalid) sm.kblk[sv][r] = kNoKeyBlk;
        if (lane < 8 && r < nvalid) dma4(src, lds_addr(&sm.kblk[sv][run0]));
        return 2 * NI + 1;
      } else {
        // With a window the keys' positions follow the same way, from the arrays beside
        // the ids.
        bool from_q = true;
        int64_t off = it.q0;
        if (r < nvalid) {
          if (!cached) {
            off = it.q0 + j;
          } else if (st.row0 >= 0) {
            from_q = false;
            off = (int64_t)st.row0 + (lane & 7);
          } else {
            int lp, slot;
            page_split(j, a.page_size, a.page_shift, &lp, &slot);
            const int p = a.page_table[(int64_t)it.s * a.max_pages + min(lp, a.max_pages - 1)];
            if (p >= 0 && p < a.num_pages) {
              from_q = false;
              off = (int64_t)p * a.page_size + slot;
            }
          }
        }
        if (lane < 8 && r >= nvalid) {
          sm.kblk[sv][r] = kNoKeyBlk;
          sm.kpos[sv][r] = 0;
        }
        if (lane < 8 && r < nvalid) {
          dma4((from_q ? a.q_blk : a.kv_blk) + off, lds_addr(&sm.kblk[sv][run0]));
          dma4((from_q ? a.q_pos : a.kv_pos) + off, lds_addr(&sm.kpos[sv][run0]));
        }
        return 2 * NI + 2;
      }
    }
  }
  return 2 * NI;
}

// First memory row of 8-row run q of each staged tile entry (see Stage): N slots per
// thread, slot k being window slot tq + k*nthr (tile slot / kWaves, run slot % kWaves).
// The page-table loads of all slots are issued together, unconditionally at a clamped
// index, so that the staging costs one memory round trip rather than one per slot.
template <int N>
__device__ __forceinline__ void run_rows(const AttnArgs& a, const Item& it, const int32_t* pt, const int (&we)[N],
                                         int tq, int nthr, int nt, int (&wr)[N]) {
  const bool grp_pages = a.page_size % kRowsPerWave == 0;
  const int cap = a.max_pages * a.page_size;
  int lp[N], slot[N], kind[N];   // kind 1: cached run, 2: live run in the pool, else wr set
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = tq + k * nthr, q = i % kWaves, vt = we[k] >> 1;
    kind[k] = 0;
    lp[k] = slot[k] = 0;
    wr[k] = -1;
    if (i < nt * kWaves) {
      if (vt < a.nct) {
        const int j0 = vt * kTileK + kRowsPerWave * q;
        if (grp_pages && j0 + kRowsPerWave <= it.kvl) {
          kind[k] = 1;
          page_split(j0, a.page_size, a.page_shift, &lp[k], &slot[k]);
        }
      } else if (a.live_in_cache) {
        const int r0 = (vt - a.nct) * kTileK + kRowsPerWave * q, j0 = it.kvl + r0;
        if (r0 + kRowsPerWave <= it.q_len && j0 + kRowsPerWave <= cap) {
          kind[k] = 2;
          page_split(j0, a.page_size, a.page_shift, &lp[k], &slot[k]);
        }
      } else {
        const int r0 = (vt - a.nct) * kTileK + kRowsPerWave * q;
        if (r0 + kRowsPerWave <= it.q_len) wr[k] = it.q0 + r0;
      }
    }
  }
  int p0[N], p1[N];
#pragma unroll
  for (int k = 0; k < N; ++k) p0[k] = pt[kind[k] ? lp[k] : 0];
#pragma unroll
  for (int k = 0; k < N; ++k) p1[k] = a.live_in_cache ? pt[kind[k] == 2 ? min(lp[k] + 1, a.max_pages - 1) : 0] : -1;
  asm volatile("" ::: "memory");   // all loads issued here, not sunk into the uses below
#pragma unroll
  for (int k = 0; k < N; ++k) {
    if (!kind[k] || p0[k] < 0 || p0[k] >= a.num_pages) continue;
    if (slot[k] + kRowsPerWave <= a.page_size) {
      wr[k] = p0[k] * a.page_size + slot[k];
    } else if (kind[k] == 2 && kRowsPerWave - (a.page_size - slot[k]) <= a.page_size &&
               lp[k] + 1 - it.lp_live < kLivePages && p1[k] >= 0 && p1[k] < a.num_pages) {
      // A live run crossing into the next page (its last row lies in page lp + 1, which
      // therefore exists): stored as -(first row) - 2.
      wr[k] = -(p0[k] * a.page_size + slot[k]) - 2;
    }
  }
}

// Wave schedule. The 8 waves form two groups, A = waves 0-3 and B = waves 4-7, one wave
// of each per SIMD. Each tile t is handled in two phases per wave: a matrix phase
// (S(t) = K(t) Q^T, then O += V(t-1) P(t-1)) and a vector phase (mask, online softmax
// of S(t) into P(t), issuing loads, waiting for its own loads). Workgroup barriers split
// time into half-steps H0, H1, ...; group A runs the matrix phase of tile t in H(2t) and
// the vector phase in H(2t+1), group B one half-step later, so on every SIMD one wave's
// matrix instructions run beside the other wave's vector instructions.
//
// Loads: a wave of group A issues its share of tile t+2 in its vector phase of tile t
// (half-step H(2t+1)), a wave of group B its share of tile t+3 (H(2t+2)); each then waits
// until only that newest tile is still in flight. So tile x is issued in H(2x-4) and
// H(2x-3) and complete and visible at the barrier that starts H(2x), when group A first
// reads it. K(x) is last read in H(2x+1), V(x) and the block ids of x in H(2x+3), all before
// the loads of tile x+3 (keys) or x+4 (values) start in H(2x+2) or later: three key
// stages and four value stages suffice.
// BAND_B: mode B with a sliding window (keys' positions staged beside their block ids).
// Kernel instances (KIND). Each lean kind pins some arguments at entry, so that the other
// paths' state and branches drop out of the tile loop, which frees registers. kLeanA: mode A
// without a window, live rows passed in (the decode and prefill shapes). kLeanB: mode B
// without a window (multi-canvas decoding). kLeanAW: mode A with a window. kLeanAL, kLeanBL:
// mode A or B without a window, live rows read from the pool. In mode A without a window the
// plan entries follow from the unit's lengths (kLeanA, kLeanAL). kGeneral: anything else (a
// window together with live rows in the pool, or mode B with a window, which has its own
// band flag).
enum : int { kGeneral = 0, kLeanA = 1, kLeanB = 2, kLeanAW = 3, kLeanAL = 4, kLeanBL = 5 };
template <int KIND>
__device__ __forceinline__ void pin_kind(AttnArgs& a) {
  if constexpr (KIND == kGeneral) return;
  constexpr bool mb = KIND == kLeanB || KIND == kLeanBL;
  a.live_in_cache = KIND == kLeanAL || KIND == kLeanBL ? 1 : 0;
  a.q_pos = a.kv_pos = nullptr;
  a.mode_b = mb ? 1 : 0;
  if constexpr (KIND != kLeanAW) a.window = 0;
  if constexpr (!mb) a.q_blk = a.kv_blk = nullptr;
}
__host__ __device__ inline int kind_of(const AttnArgs& a, bool band_b) {
  if (band_b) return kGeneral;
  if (a.live_in_cache) return a.window != 0 ? kGeneral : a.mode_b ? kLeanBL : kLeanAL;
  if (a.mode_b) return a.window == 0 ? kLeanB : kGeneral;
  return a.window == 0 ? kLeanA : kLeanAW;
}

template <int HD, bool BAND_B, int KIND>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnArgs a) {
  constexpr bool LEAN = KIND == kLeanA || KIND == kLeanAL;   // plan entries from the lengths
  pin_kind<KIND>(a);
  using D = DmaShape<HD>;
  constexpr int NI = D::NI;
  constexpr int NT = HD / 16;       // MFMA steps over d for the scores
  constexpr int NDB = HD / 32;      // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) AttnSmem<HD> sm;
  // LDS byte addresses of the first key and value stages.
  const unsigned k_lds0 = lds_addr(&sm.k[0][0]), v_lds0 = lds_addr(&sm.v[0][0]);
  constexpr unsigned kKStageBytes = sizeof(sm.k[0]), kVStageBytes = sizeof(sm.v[0]);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hl = lane >> 5;
  const int grp = uni(wave) >> 2;   // 0: group A, 1: group B (scalar: guards barriers)
  const int lead = 2 + grp;         // tiles ahead of the current one that this wave issues
  const int G = a.G;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt, a.Hkv);
  cint32* plan = as_const(a.plan);
  // The range's record holds its item bounds and a copy of its first item.
  cint32* rec = plan + L.rng + kRngWords * range_of_wg(blockIdx.x);   // in bounds for any plan
  const int w_begin = rec[0], w_end = rec[1];
  {
    // The record and the header arrive in one round trip; the check follows.
    PlanShape h = plan_shape(plan);
    asm volatile("" : "+s"(h.w[0]), "+s"(h.w[1]), "+s"(h.w[2]), "+s"(h.w[3]), "+s"(h.w[4]), "+s"(h.w[5]), "+s"(h.w[6]),
                 "+s"(h.w[7]), "+s"(h.w[8]), "+s"(h.w[9]), "+s"(h.w[10]), "+s"(h.w[11]) : "s"(w_begin), "s"(w_end));
    if (!plan_matches(h, a)) return;
  }
  const uint16_t* qg = (const uint16_t*)a.q;
  const float sl2 = a.scale_log2;
  // V transpose reads: lane (group g16 = lane/16, j = lane%16) is source lane 4*ta + tc of
  // its group: it reads 8 bytes of row 4*(lane/32) + ta (+8 for the second half of the
  // step) at d = 16*(g16%2) + 4*tc, and receives d = lane%32 for 4 keys.
  const int ta = (lane & 15) >> 2, tc = lane & 3;
  const int vrow0 = 4 * hl + ta;
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * tc;
  const int rho = wave * 32 + col;           // this lane's packed query row
  // LDS operand offsets (elements). The K swizzle of rows 32kb+col does not depend on kb,
  // so step t of either key block reads at koff[t] (+32 rows for kb = 1). The V swizzle of
  // the rows a lane reads is the same for every (kb, hs, +8) step, so block db reads at
  // voff[db] plus a constant row offset.
  int koff[HD / 16], voff[HD / 32];
  {
    const int sw = kswz<HD>(col);
#pragma unroll
    for (int t = 0; t < HD / 16; ++t) koff[t] = col * HD + 8 * ((2 * t + hl) ^ sw);
    const int vs = vswz<HD>(vrow0);
#pragma unroll
    for (int db = 0; db < HD / 32; ++db) {
      const int dcol = 32 * db + vcol0;
      voff[db] = vrow0 * HD + ((dcol >> 3) ^ vs) * 8 + (dcol & 7);
    }
  }
  FastOffsets<HD> fo;
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int rr = k * D::RPI + lane / D::CPR, r = kRowsPerWave * wave + rr, pch = lane % D::CPR;
    fo.k[k] = (unsigned)(((int64_t)rr * a.Hkv * HD + 8 * (pch ^ kswz<HD>(r))) * 2);
    fo.v[k] = (unsigned)(((int64_t)rr * a.Hkv * HD + 8 * (pch ^ vswz<HD>(r))) * 2);
  }
  if (a.stats && blockIdx.x == 0 && tid == 0)   // skipped tiles of the whole grid, per kv head
    atomicAdd(&a.stats[2], (unsigned long long)a.Hkv * ((unsigned long long)L.units * a.nkt - plan[3]));

  for (int item = w_begin; item < w_end; ++item) {
    Item it;
    cint32* ip = item == w_begin ? rec + 2 : plan + L.items + kItemWords * (int64_t)item;
    PlanItem pi;
    read_item(ip, &pi);
    const int u = pi.u, ob = pi.ob, oe = pi.oe, pslot = pi.pslot;
    it.g = pi.g;
    it.s = u / a.nqt;
    const int r = u - it.s * a.nqt;
    it.q0 = pi.q0;       // the unit's live rows and committed length, as the planner
    it.q_len = pi.q_len; // clamped them
    it.kvl = pi.kvl;
    it.lp_live = a.page_shift >= 0 ? it.kvl >> a.page_shift : it.kvl / a.page_size;
    const int i0 = r * a.tile_q;
    const int32_t* list = a.plan + L.list + (int64_t)u * a.nkt;

    // The item's tiles are processed in windows: the window's plan entries and the pages of
    // its cached tiles are staged in LDS first, so the tile loop reads its metadata from
    // LDS only and issues no memory loads but the tiles' own. Thread tid stages window slots
    // tid + k * kThreads (tile slot / 8, wave slot % 8); the loads come in two rounds (plan
    // entries, then page-table entries), issued apart from the LDS writes so that the first
    // window's rounds overlap the query loads.
    const int32_t* pt = a.page_table + (int64_t)it.s * a.max_pages;
    int we[kWinPerThread], wr[kWinPerThread];
    int tq = tid;
    asm volatile("" : "+v"(tq));   // slot math stays here, not hoisted out of the item loop
    auto win_load_entries = [&](int wb, int nt) {
      if constexpr (LEAN) {
        // Mode A without a window: the entries follow from the unit's lengths, with no load.
        const int nc = mode_a_cached(a, it), qmin = i0 / a.block_size;
#pragma unroll
        for (int k = 0; k < kWinPerThread; ++k) {
          const int i = tq + k * kThreads;
          we[k] = i < nt * kWaves ? mode_a_entry(a, it, nc, qmin, wb + i / kWaves) : 0;
        }
      } else {
#pragma unroll
        for (int k = 0; k < kWinPerThread; ++k) {
          const int i = tq + k * kThreads;
          we[k] = i < nt * kWaves ? list[wb + i / kWaves] : 0;
        }
      }
    };
    auto win_load_rows = [&](int nt) { run_rows<kWinPerThread>(a, it, pt, we, tq, kThreads, nt, wr); };
    win_load_entries(ob, min(oe - ob, kWin));
    // Live rows in the pool: the pages of their logical pages lp_live, lp_live+1, ...
    int lpg = -1;
    if (a.live_in_cache && tq < kLivePages && it.lp_live + tq < a.max_pages) lpg = pt[it.lp_live + tq];
    asm volatile("" ::: "memory");   // keep the plan-entry loads ahead of the query loads

    // Query fragments of this lane's column (B operand of S^T = K Q^T), held in registers
    // for the whole item; padding rows read zeros.
    const int pos = i0 + rho / G, hh = rho - (rho / G) * G;
    const bool qvalid = pos < it.q_len;
    bf16x8 qf[NT];
    {
      const uint16_t* qp = qg + ((int64_t)(it.q0 + pos) * a.Hq + (int64_t)it.g * G + hh) * HD + 8 * hl;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 z = {};
        qf[t] = qvalid ? *(const bf16x8*)(qp + 16 * t) : z;
      }
    }
    const int qblk = !qvalid ? kNoKeyBlk - 1 : (a.mode_b ? a.q_blk[it.q0 + pos] : pos / a.block_size);
    int qpos = 0;
    if constexpr (BAND_B) qpos = qvalid ? a.q_pos[it.q0 + pos] : 0;
    asm volatile("" ::: "memory");   // the page-table loads follow the query loads
    win_load_rows(min(oe - ob, kWin));

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float m = 0.f, l = 0.f;   // reference and row sum of the online softmax (tile_softmax)
    int n_partial = 0;

    for (int wb = ob; wb < oe; wb += kWin) {
      const int nt = min(oe - wb, kWin);     // tiles in this window
      if (wb != ob) {
        win_load_entries(wb, nt);
        win_load_rows(nt);
      }
      __syncthreads();   // earlier readers of LDS (previous window or item) are finished
#pragma unroll
      for (int k = 0; k < kWinPerThread; ++k) {
        const int i = tq + k * kThreads, ti = i / kWaves, q = i % kWaves;
        if (i < nt * kWaves) {
          if (q == 0) sm.win_e[ti] = we[k];
          sm.win_row[ti][q] = wr[k];
        }
      }
      if (a.live_in_cache && wb == ob && tq < kLivePages) sm.live_pg[tq] = lpg;
      __syncthreads();
      // The query loads were issued before the page-table loads just waited for, so they
      // have landed: no wait for them falls inside the tile loop (where it would also wait
      // for every tile in flight).
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" ::"v"(qf[t]));
      asm volatile("" ::"v"(qblk));
      if constexpr (BAND_B) asm volatile("" ::"v"(qpos));

      // Prologue: tiles 0 .. lead-1 issued; this wave waits for all of them but the last
      // (group A: tile 0; group B: tiles 0 and 1), then tile 0 is published.
      int issued = 0;
      for (int x = 0; x < lead; ++x) {
        const Stage st = meta_resolve(meta_read(x, nt, wave, sm));
        issued = stage_fetch<HD, NI, BAND_B>(a, it, st, sm, x % kKStages, x % kVStages, k_lds0 + (x % kKStages) * kKStageBytes,
                                             v_lds0 + (x % kVStages) * kVStageBytes, fo, uni(wave));
      }
      // Stages of tile lead, the next to issue, advanced by one per vector phase.
      int xk = lead % kKStages, xv = lead % kVStages;
      RawMeta raw = meta_read(lead, nt, wave, sm);         // next tile to issue
      int e_next = sm.win_e[0];                            // entry of the next tile to mask
      wait_vm(issued);
      __syncthreads();
      if (grp) __syncthreads();           // group B starts half a step later

      bf16x8 pf[2][2];
      f32x16 sc[2];
      // Matrix phase: O^T += V^T P^T for tile t-1 (when WITH_PV), then S^T(t) = K Q^T for
      // two 32-key blocks x this wave's 32 query columns (when WITH_S). Operand reads run a
      // few steps ahead of the matrix instructions that consume them.
      auto matrix_phase = [&](int t, auto with_s, auto with_pv) {
        constexpr bool WITH_S = decltype(with_s)::value, WITH_PV = decltype(with_pv)::value;
        if constexpr (WITH_PV) {
          // Step (kb, hs) covers keys 32kb+16hs .. +15; lane half hl feeds the keys
          // 32kb+16hs + {4hl..4hl+3, 8+4hl..8+4hl+3} (its score registers), which two
          // transpose reads deliver as the A operand, for d = 32db + lane%32.
          const uint16_t* vt = sm.v[(t - 1) % kVStages];
          bf16x8 vf[2][2][NDB];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                const int rofs = (32 * kb + 16 * hs) * HD;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[voff[db] + rofs]);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[voff[db] + rofs + 8 * HD]);
                vf[kb][hs][db] = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
              for (int db = 0; db < NDB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb][hs][db], pf[kb][hs], o[db], 0, 0, 0);
        }
        if constexpr (WITH_S) {
          const uint16_t* kt = sm.k[t % kKStages];
          bf16x8 kf[NT][2];
#pragma unroll
          for (int s = 0; s < NT; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) kf[s][kb] = *(const bf16x8*)&kt[koff[s] + 32 * kb * HD];
#pragma unroll
          for (int s = 0; s < NT; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)      // alternate the two accumulators
              sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s][kb], qf[s], s == 0 ? f32x16{} : sc[kb], 0, 0, 0);
        }
        // Interleave: ten operand reads first, then one matrix instruction per read
        // (K: one b128 read per instruction; V: two transpose reads per instruction).
        constexpr int NR = (WITH_S ? 2 * NT : 0) + (WITH_PV ? 8 * NDB : 0);
        constexpr int NM = (WITH_S ? 2 * NT : 0) + (WITH_PV ? 4 * NDB : 0);
        constexpr int AHEAD = NR < 10 ? NR : 10;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
        interleave<NM, NR, AHEAD>();
      };

      // Vector phase of tile t: issue this wave's loads of tile t+lead and read the metadata
      // of the tile after it, then mask (partial tiles only) and the online softmax of S(t)
      // into P(t), then wait until only the tile just issued is in flight.
      auto vector_phase = [&](int t) {
        {
          const int x = t + lead;
          // The loads go out at the matrix phase's priority, ahead of the other wave's
          // instructions, so that they start their HBM round trip as early as possible.
          __builtin_amdgcn_s_setprio(1);
          issued = stage_fetch<HD, NI, BAND_B>(a, it, meta_resolve(raw), sm, xk, xv, k_lds0 + xk * kKStageBytes,
                                               v_lds0 + xv * kVStageBytes, fo, uni(wave));
          __builtin_amdgcn_s_setprio(0);
          raw = meta_read(x + 1, nt, wave, sm);
          xk = xk == kKStages - 1 ? 0 : xk + 1;
          xv = xv == kVStages - 1 ? 0 : xv + 1;
        }
        const int e_t = uni(e_next);
        e_next = sm.win_e[min(t + 1, kWin - 1)];   // used next phase, only if t+1 < nt
        // Lane (col, hl) holds key 32kb + 8(v/4) + 4hl + v%4.
        const bool partial = e_t & 1;
        n_partial += partial;
        if (partial) {   // absent keys carry kNoKeyBlk, which no row sees
          const int* kbl = sm.kblk[t % kVStages] + 4 * hl;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
              const i32x4 kbw = *(const i32x4*)&kbl[32 * kb + 8 * v4];
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (kbw[c] > qblk) sc[kb][4 * v4 + c] = -INFINITY;
            }
          if (a.window > 0 && !a.mode_b) {
            // Sliding window (mode A): the key in column cc of the tile lies wbase - cc
            // positions before this lane's query (committed row j at position j, live row
            // i at kv_len + i); it drops out once that distance reaches the window.
            const int vt = e_t >> 1;
            const int wbase = pos + (vt < a.nct ? it.kvl - vt * kTileK : -(vt - a.nct) * kTileK);
            const int thr = wbase - a.window - 4 * hl;   // mask 32kb + 8(v/4) + v%4 <= thr
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if (32 * kb + 8 * (v / 4) + v % 4 <= thr) sc[kb][v] = -INFINITY;
          } else if constexpr (BAND_B) {
            // Sliding window (mode B): the keys' positions were staged beside their ids.
            const int* kpl = sm.kpos[t % kVStages] + 4 * hl;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4) {
                const i32x4 kpw = *(const i32x4*)&kpl[32 * kb + 8 * v4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if ((int64_t)qpos - kpw[c] >= a.window) sc[kb][4 * v4 + c] = -INFINITY;
              }
          }
        }
        tile_softmax<NDB>(sc, sl2, m, l, o, pf);
        // Keep the softmax ahead of the wait below (the compiler may not sink it past).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) asm volatile("" ::"v"(pf[kb][hs]));
        asm volatile("" ::"v"(l));
        wait_vm(issued);
      };

      __builtin_amdgcn_s_setprio(1);
      matrix_phase(0, std::true_type{}, std::false_type{});
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      vector_phase(0);
      __syncthreads();
      for (int t = 1; t < nt; ++t) {
        // The wave in its matrix phase takes the SIMD's issue arbitration from the wave in its
        // vector phase (here and in the item's first and last matrix phase), so that the matrix
        // instructions of the younger group are not held behind the older group's softmax; the
        // four phases then last about as long.
        __builtin_amdgcn_s_setprio(1);
        matrix_phase(t, std::true_type{}, std::true_type{});
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        vector_phase(t);
        __syncthreads();
      }
      // The last tile's PV product; group A then waits out group B's last vector phase.
      __builtin_amdgcn_s_setprio(1);
      matrix_phase(nt, std::false_type{}, std::true_type{});
      __builtin_amdgcn_s_setprio(0);
      if (!grp) __syncthreads();
    }   // window

    // Epilogue. Lane (col, hl) of block db holds d = 32db + 8(v/4) + 4hl + v%4 of packed
    // row rho. Each pass writes one 128-byte column segment of the wave's 32 rows into the
    // wave's staging area (16-byte chunk c of row r at chunk c ^ (r & 7)) and reads it back
    // as 8 rows x 128 bytes per instruction, so every store covers whole row segments.
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = lt > 0.f ? m + __log2f(lt) : -INFINITY;
    float* ep = sm.ep[wave];
    // Per-lane index math is recomputed here rather than hoisted out of the item loop,
    // where it would only hold registers.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int ec = ln & 7;                         // read-back chunk of this lane
    const int ecol = ln & 31, ehl = ln >> 5;       // = col, hl
    int brow[4];                                   // memory row of each read-back row, -1: none
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = wave * 32 + 8 * k + (ln >> 3), pr = i0 + rr / G, hr = rr - (rr / G) * G;
      brow[k] = pr >= it.q_len ? -1
                : pslot < 0 ? (it.q0 + pr) * a.Hq + it.g * G + hr
                            : pslot * kRowsPerWG + rr;
    }
    auto ep_slot = [&](int r, int c) { return r * (kEpRowBytes / 4) + 4 * (c ^ (r & 7)); };
    // All passes' LDS writes and reads are issued before the first store, so the LDS round
    // trips overlap; the wave's LDS accesses execute in order, so a pass's writes land
    // after the previous pass's reads.
    if (pslot < 0) {
      uint16_t* op = (uint16_t*)a.out;
      bf16x8 y[NDB / 2][4];
#pragma unroll
      for (int pb = 0; pb < NDB / 2; ++pb) {     // 64 bf16 values per row and pass
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x16& ob16 = o[2 * pb + j];
            f32x4 x = {ob16[4 * v4] * inv, ob16[4 * v4 + 1] * inv, ob16[4 * v4 + 2] * inv, ob16[4 * v4 + 3] * inv};
            *(bf16x4*)&ep[ep_slot(ecol, 4 * j + v4) + 2 * ehl] = __builtin_convertvector(x, bf16x4);
          }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 4; ++k) y[pb][k] = *(const bf16x8*)&ep[ep_slot(8 * k + (ln >> 3), ec)];
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int pb = 0; pb < NDB / 2; ++pb)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (brow[k] >= 0) *(bf16x8*)(op + (int64_t)brow[k] * HD + 64 * pb + 8 * ec) = y[pb][k];
      if (qvalid && ehl == 0 && a.lse) {
        const int pe = i0 + (wave * 32 + ecol) / G, he = wave * 32 + ecol - ((wave * 32 + ecol) / G) * G;
        a.lse[(int64_t)(it.q0 + pe) * a.Hq + (int64_t)it.g * G + he] = lse2 * kLn2;
      }
    } else {
      // A split piece: fp16 partial rows (piece_factor) through the same staging.
      float amax = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(o[db][v]));
      float restore;
      const float mul = piece_factor(amax, inv, &restore);
      f16x8 y[NDB / 2][4];
#pragma unroll
      for (int pb = 0; pb < NDB / 2; ++pb) {     // 64 fp16 values per row and pass
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const f32x16& ob16 = o[2 * pb + j];
            f32x4 x = {ob16[4 * v4] * mul, ob16[4 * v4 + 1] * mul, ob16[4 * v4 + 2] * mul, ob16[4 * v4 + 3] * mul};
            *(f16x4*)&ep[ep_slot(ecol, 4 * j + v4) + 2 * ehl] = __builtin_convertvector(x, f16x4);
          }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 4; ++k) y[pb][k] = *(const f16x8*)&ep[ep_slot(8 * k + (ln >> 3), ec)];
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int pb = 0; pb < NDB / 2; ++pb)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (brow[k] >= 0) *(f16x8*)(a.part_h + (int64_t)brow[k] * HD + 64 * pb + 8 * ec) = y[pb][k];
      if (qvalid && ehl == 0) {
        a.part_lse[pslot * kRowsPerWG + wave * 32 + ecol] = lse2;
        a.part_scale[pslot * kRowsPerWG + wave * 32 + ecol] = restore;
      }
    }

    if (a.stats && tid == 0) {
      const int n = oe - ob;
      // n_partial counts the tiles of wave 0 only: every wave sees every tile.
      atomicAdd(&a.stats[0], (unsigned long long)(n - n_partial));
      atomicAdd(&a.stats[1], (unsigned long long)n_partial);
      atomicAdd(&a.stats[3], (unsigned long long)n * 2ull * kTileK * HD * 2ull);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Narrow items: live blocks of at most 64 packed rows per (sequence, kv head), such as a
// short causal extend of up to 16 positions at four query heads per kv head.
//
// With so few live rows the wide kernel's 256-row work items would be mostly padding while
// each key tile still costs the full matrix and softmax work. Here a workgroup of four waves
// owns an item of 64 packed rows. The waves form two teams of two (one wave per SIMD), each
// wave of a team holding 32 rows; team p computes the tiles p, p+2, p+4, ... of each window
// with its own online-softmax state, so two tiles are in work at once, and team 1's state is
// merged into team 0's at the end. Every wave stages two of each tile's eight 8-row runs into
// a ring of four stages, one pair of tiles ahead of the pair in work: a barrier before a
// pair's loads frees the two stages they overwrite (every wave is done with the pair before),
// and one after them publishes the pair in work (each wave has waited for its own loads).
constexpr int kNWaves = 4, kNThreads = 64 * kNWaves;
constexpr int kNStages = 4;                           // two pairs of tiles
constexpr int kNRuns = kWaves / kNWaves;              // 8-row runs each wave stages per tile
constexpr int kNWinPerThread = kWin * kWaves / kNThreads;

template <int HD>
struct NarrowSmem {
  uint16_t k[kNStages][kTileK * HD];
  uint16_t v[kNStages][kTileK * HD];
  int kblk[kNStages][kTileK];
  int kpos[kNStages][kTileK];
  int win_e[kWin];
  int win_row[kWin][kWaves];       // per tile and 8-row run, as in the wide kernel
  int live_pg[kLivePages];
};

// s_waitcnt vmcnt(n) for a wave-uniform n in [LO, HI], by binary search over immediates.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_in(int n) {
  if constexpr (LO == HI) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LO) : "memory");
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vm_in<LO, MID>(n);
    else wait_vm_in<MID + 1, HI>(n);
  }
}

template <int HD, bool BAND_B, int KIND>
__global__ __launch_bounds__(kNThreads) void attn_bf16_narrow_kernel(AttnArgs a) {
  constexpr bool LEAN = KIND == kLeanA || KIND == kLeanAL;   // plan entries from the lengths
  pin_kind<KIND>(a);
  using D = DmaShape<HD>;
  constexpr int NI = D::NI;
  constexpr int NT = HD / 16, NDB = HD / 32;
  // Loads in flight per wave stay within the 6-bit counter: two pairs of tiles.
  static_assert(4 * kNRuns * (2 * NI + 2) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) NarrowSmem<HD> sm;
  const unsigned k_lds0 = lds_addr(&sm.k[0][0]), v_lds0 = lds_addr(&sm.v[0][0]);
  constexpr unsigned kNStageBytes = sizeof(sm.k[0]);
  static_assert(sizeof(sm.k[0]) == sizeof(sm.v[0]), "one stage size for keys and values");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hl = lane >> 5;
  const int team = uni(wave) >> 1;           // computes tiles team, team + 2, ... of a window
  const int G = a.G;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt, a.Hkv);
  cint32* plan = as_const(a.plan);
  cint32* rec = plan + L.rng + kRngWords * range_of_wg(blockIdx.x);   // in bounds for any plan
  const int w_begin = rec[0], w_end = rec[1];
  {
    // The record and the header arrive in one round trip; the check follows.
    PlanShape h = plan_shape(plan);
    asm volatile("" : "+s"(h.w[0]), "+s"(h.w[1]), "+s"(h.w[2]), "+s"(h.w[3]), "+s"(h.w[4]), "+s"(h.w[5]), "+s"(h.w[6]),
                 "+s"(h.w[7]), "+s"(h.w[8]), "+s"(h.w[9]), "+s"(h.w[10]), "+s"(h.w[11]) : "s"(w_begin), "s"(w_end));
    if (!plan_matches(h, a)) return;
  }
  const uint16_t* qg = (const uint16_t*)a.q;
  const float sl2 = a.scale_log2;
  const int ta = (lane & 15) >> 2, tc = lane & 3;
  const int vrow0 = 4 * hl + ta;
  const int vcol0 = 16 * ((lane >> 4) & 1) + 4 * tc;
  const int rho = (wave & 1) * 32 + col;     // this lane's packed query row (in either team)
  int koff[NT], voff[NDB];
  {
    const int sw = kswz<HD>(col);
#pragma unroll
    for (int t = 0; t < NT; ++t) koff[t] = col * HD + 8 * ((2 * t + hl) ^ sw);
    const int vs = vswz<HD>(vrow0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dcol = 32 * db + vcol0;
      voff[db] = vrow0 * HD + ((dcol >> 3) ^ vs) * 8 + (dcol & 7);
    }
  }
  // Fast-path offsets for runs of even and odd index (the K swizzle depends on the parity).
  FastOffsets<HD> fo[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int rr = k * D::RPI + lane / D::CPR, r = kRowsPerWave * par + rr, pch = lane % D::CPR;
      fo[par].k[k] = (unsigned)(((int64_t)rr * a.Hkv * HD + 8 * (pch ^ kswz<HD>(r))) * 2);
      fo[par].v[k] = (unsigned)(((int64_t)rr * a.Hkv * HD + 8 * (pch ^ vswz<HD>(r))) * 2);
    }
  if (a.stats && blockIdx.x == 0 && tid == 0)
    atomicAdd(&a.stats[2], (unsigned long long)a.Hkv * ((unsigned long long)L.units * a.nkt - plan[3]));

  for (int item = w_begin; item < w_end; ++item) {
    Item it;
    cint32* ip = item == w_begin ? rec + 2 : plan + L.items + kItemWords * (int64_t)item;
    PlanItem pi;
    read_item(ip, &pi);
    const int u = pi.u, ob = pi.ob, oe = pi.oe, pslot = pi.pslot;
    it.g = pi.g;
    it.s = u / a.nqt;
    const int r = u - it.s * a.nqt;
    it.q0 = pi.q0;
    it.q_len = pi.q_len;
    it.kvl = pi.kvl;
    it.lp_live = a.page_shift >= 0 ? it.kvl >> a.page_shift : it.kvl / a.page_size;
    const int i0 = r * a.tile_q;
    const int32_t* list = a.plan + L.list + (int64_t)u * a.nkt;
    const int32_t* pt = a.page_table + (int64_t)it.s * a.max_pages;

    // Window staging, as in the wide kernel: plan entries, then the first memory row of
    // every 8-row run of every tile (-1: general path; <= -2: a live run crossing a page).
    auto win_stage = [&](int wb, int nt) {
      int we[kNWinPerThread], wr[kNWinPerThread];
      const int nc = mode_a_cached(a, it), qmin = i0 / a.block_size;   // (lean instance)
#pragma unroll
      for (int k = 0; k < kNWinPerThread; ++k) {
        const int i = tid + k * kNThreads;
        if constexpr (LEAN) we[k] = i < nt * kWaves ? mode_a_entry(a, it, nc, qmin, wb + i / kWaves) : 0;
        else we[k] = i < nt * kWaves ? list[wb + i / kWaves] : 0;
      }
      run_rows<kNWinPerThread>(a, it, pt, we, tid, kNThreads, nt, wr);
      __syncthreads();   // earlier readers of the window (previous window or item) are done
#pragma unroll
      for (int k = 0; k < kNWinPerThread; ++k) {
        const int i = tid + k * kNThreads, ti = i / kWaves, q = i % kWaves;
        if (i < nt * kWaves) {
          if (q == 0) sm.win_e[ti] = we[k];
          sm.win_row[ti][q] = wr[k];
        }
      }
    };

    // Query fragments and block id of this lane's row.
    const int pos = i0 + rho / G, hh = rho - (rho / G) * G;
    const bool qvalid = rho < a.tile_q * G && pos < it.q_len;
    bf16x8 qf[NT];
    {
      const uint16_t* qp = qg + ((int64_t)(it.q0 + pos) * a.Hq + (int64_t)it.g * G + hh) * HD + 8 * hl;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 z = {};
        qf[t] = qvalid ? *(const bf16x8*)(qp + 16 * t) : z;
      }
    }
    const int qblk = !qvalid ? kNoKeyBlk - 1 : (a.mode_b ? a.q_blk[it.q0 + pos] : pos / a.block_size);
    int qpos = 0;
    if constexpr (BAND_B) qpos = qvalid ? a.q_pos[it.q0 + pos] : 0;
    int lpg[(kLivePages + kNThreads - 1) / kNThreads];
#pragma unroll
    for (int k = 0; k < (kLivePages + kNThreads - 1) / kNThreads; ++k) {
      const int i = tid + k * kNThreads;
      lpg[k] = a.live_in_cache && i < kLivePages && it.lp_live + i < a.max_pages ? pt[it.lp_live + i] : -1;
    }

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float m = -INFINITY, l = 0.f;
    int n_partial = 0, n_mine = 0;

    for (int wb = ob; wb < oe; wb += kWin) {
      const int nt = min(oe - wb, kWin);
      win_stage(wb, nt);
      if (wb == ob) {
#pragma unroll
        for (int k = 0; k < (kLivePages + kNThreads - 1) / kNThreads; ++k) {
          const int i = tid + k * kNThreads;
          if (i < kLivePages) sm.live_pg[i] = lpg[k];
        }
      }
      __syncthreads();

      // This wave's two runs of tile x into stage x % kNStages; returns the loads issued.
      auto fetch = [&](int x) {
        int n = 0;
#pragma unroll
        for (int j = 0; j < kNRuns; ++j) {
          const int q = uni(wave) * kNRuns + j;
          const Stage st = meta_resolve(meta_read(x, nt, q, sm));
          const int sx = x % kNStages;
          n += stage_fetch<HD, NI, BAND_B>(a, it, st, sm, sx, sx, k_lds0 + sx * kNStageBytes, v_lds0 + sx * kNStageBytes,
                                           fo[j & 1], q);
        }
        return n;
      };
      fetch(0);
      fetch(1);
      for (int k = 0; 2 * k < nt; ++k) {
        __syncthreads();               // every wave is done with pair k-1: its stages are free
        int cnext = 0;                 // this wave's loads of pair k+1
        if (2 * k + 2 < nt) cnext += fetch(2 * k + 2);
        if (2 * k + 3 < nt) cnext += fetch(2 * k + 3);
        wait_vm_in<0, 63>(cnext);      // this wave's loads of pair k have landed
        __syncthreads();               // and every other wave's
        const int t = 2 * k + team;
        if (t >= nt) continue;         // an odd last tile: team 1 has none
        const int e_t = uni(sm.win_e[t]);
        const int st_ = t % kNStages;
        ++n_mine;

        // S^T = K Q^T for this wave's 32 rows (two 32-key blocks).
        f32x16 sc[2];
        {
          const uint16_t* kt = sm.k[st_];
#pragma unroll
          for (int s = 0; s < NT; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const bf16x8 kf = *(const bf16x8*)&kt[koff[s] + 32 * kb * HD];
              sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], s == 0 ? f32x16{} : sc[kb], 0, 0, 0);
            }
        }
        // Mask (partial tiles only) as in the wide kernel, then the online softmax with a
        // lazy reference max: m moves only when a row's max grows by more than 2^8 (or on
        // its first visible key). This kernel's per-tile chain (scores, softmax, PV) is
        // latency-bound, and the row-sum check of tile_softmax measured slower here.
        const bool partial = e_t & 1;
        n_partial += partial;
        if (partial) {
          const int* kbl = sm.kblk[st_] + 4 * hl;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
              const i32x4 kbw = *(const i32x4*)&kbl[32 * kb + 8 * v4];
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (kbw[c] > qblk) sc[kb][4 * v4 + c] = -INFINITY;
            }
          if (a.window > 0 && !a.mode_b) {
            const int vt = e_t >> 1;
            const int wbase = pos + (vt < a.nct ? it.kvl - vt * kTileK : -(vt - a.nct) * kTileK);
            const int thr = wbase - a.window - 4 * hl;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if (32 * kb + 8 * (v / 4) + v % 4 <= thr) sc[kb][v] = -INFINITY;
          } else if constexpr (BAND_B) {
            // Sliding window (mode B): the keys' positions were staged beside their ids.
            const int* kpl = sm.kpos[st_] + 4 * hl;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4) {
                const i32x4 kpw = *(const i32x4*)&kpl[32 * kb + 8 * v4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if ((int64_t)qpos - kpw[c] >= a.window) sc[kb][4 * v4 + c] = -INFINITY;
              }
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][v]);
        mx = half_max(mx);
        const float mcand = mx * sl2;
        const bool grow = mcand > m + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float alpha = grow ? __builtin_amdgcn_exp2f(m - mcand) : 1.f;
          m = grow ? mcand : m;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        }
        const float muse = m == -INFINITY ? 0.f : m;
        bf16x8 pf[2][2];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * hs + e], sl2, -muse));
            pf[kb][hs] = to_bf16x8(x);
            rs += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
          }
        l += rs;
        // O^T += V^T P^T: step (kb, hs) covers keys 32kb+16hs .. +15 (see the wide kernel).
        {
          const uint16_t* vt = sm.v[st_];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                const int rofs = (32 * kb + 16 * hs) * HD;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[voff[db] + rofs]);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[voff[db] + rofs + 8 * HD]);
                const bf16x8 vf = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hs], o[db], 0, 0, 0);
              }
        }
      }
    }   // window

    // Merge team 1's state into team 0's through LDS (the ring is free once every wave has
    // passed this barrier): both teams hold the same rows in the same lane layout.
    __syncthreads();
    {
      constexpr int XW = NDB * 16 + 2;   // floats per lane: O, m, l
      float* xb = (float*)&sm.k[0][0] + ((wave & 1) * 64 + lane) * XW;
      if (team == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) xb[16 * db + v] = o[db][v];
        xb[NDB * 16] = m;
        xb[NDB * 16 + 1] = l;
      }
      __syncthreads();
      if (team == 0) {
        const float m1 = xb[NDB * 16], l1 = xb[NDB * 16 + 1];
        const float M = fmaxf(m, m1);
        const float a0 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        const float a1 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][v] = o[db][v] * a0 + xb[16 * db + v] * a1;
        l = l * a0 + l1 * a1;
        m = M;
      }
    }

    // Epilogue (team 0): lane (col, hl) of block db holds d = 32db + 8(v/4) + 4hl + v%4 of
    // row rho.
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = lt > 0.f ? m + __log2f(lt) : -INFINITY;
    float prestore = 1.f, pmul = inv;
    if (pslot >= 0) {   // uniform; both lane halves of a row take part in the row's maximum
      float amax = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(o[db][v]));
      pmul = piece_factor(amax, inv, &prestore);
    }
    if (qvalid && team == 0) {
      if (pslot < 0) {
        const int64_t row = (int64_t)(it.q0 + pos) * a.Hq + (int64_t)it.g * G + hh;
        uint16_t* op = (uint16_t*)a.out + row * HD + 4 * hl;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            f32x4 x = {o[db][4 * v4] * inv, o[db][4 * v4 + 1] * inv, o[db][4 * v4 + 2] * inv, o[db][4 * v4 + 3] * inv};
            *(bf16x4*)(op + 32 * db + 8 * v4) = __builtin_convertvector(x, bf16x4);
          }
        if (hl == 0 && a.lse) a.lse[row] = lse2 * kLn2;
      } else {
        // A split piece: fp16 partial row (piece_factor, taken for every lane above).
        uint16_t* pp = a.part_h + ((int64_t)pslot * kRowsPerWG + rho) * HD + 4 * hl;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            f32x4 x = {o[db][4 * v4] * pmul, o[db][4 * v4 + 1] * pmul, o[db][4 * v4 + 2] * pmul, o[db][4 * v4 + 3] * pmul};
            *(f16x4*)(pp + 32 * db + 8 * v4) = __builtin_convertvector(x, f16x4);
          }
        if (hl == 0) {
          a.part_lse[(int64_t)pslot * kRowsPerWG + rho] = lse2;
          a.part_scale[(int64_t)pslot * kRowsPerWG + rho] = prestore;
        }
      }
    }
    if (a.stats && (tid & 127) == 0) {   // the first wave of each team, for its tiles
      atomicAdd(&a.stats[0], (unsigned long long)(n_mine - n_partial));
      atomicAdd(&a.stats[1], (unsigned long long)n_partial);
      if (team == 0) atomicAdd(&a.stats[3], (unsigned long long)(oe - ob) * 2ull * kTileK * HD * 2ull);
    }
  }
}

}  // namespace

// One launcher per kernel: the head_dim, the mode-B band flag and the instance kind pick the
// template instance.
#define BCP_LAUNCH_KIND(KERNEL, HD, THREADS)                                                             \
  switch (kind) {                                                                                       \
    case kLeanA: hipLaunchKernelGGL((KERNEL<HD, false, kLeanA>), g, dim3(THREADS), 0, stream, a); break;   \
    case kLeanB: hipLaunchKernelGGL((KERNEL<HD, false, kLeanB>), g, dim3(THREADS), 0, stream, a); break;   \
    case kLeanAW: hipLaunchKernelGGL((KERNEL<HD, false, kLeanAW>), g, dim3(THREADS), 0, stream, a); break; \
    case kLeanAL: hipLaunchKernelGGL((KERNEL<HD, false, kLeanAL>), g, dim3(THREADS), 0, stream, a); break; \
    case kLeanBL: hipLaunchKernelGGL((KERNEL<HD, false, kLeanBL>), g, dim3(THREADS), 0, stream, a); break; \
    default:                                                                                            \
      if (band_b) hipLaunchKernelGGL((KERNEL<HD, true, kGeneral>), g, dim3(THREADS), 0, stream, a);      \
      else hipLaunchKernelGGL((KERNEL<HD, false, kGeneral>), g, dim3(THREADS), 0, stream, a);            \
  }

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  const bool band_b = a.mode_b && a.window > 0;
  const int kind = kind_of(a, band_b);
  const dim3 g(grid);
  if (head_dim == 128) {
    BCP_LAUNCH_KIND(attn_bf16_kernel, 128, kThreads)
  } else {
    BCP_LAUNCH_KIND(attn_bf16_kernel, 64, kThreads)
  }
  return hipGetLastError();
}

hipError_t launch_attn_bf16_narrow(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  const bool band_b = a.mode_b && a.window > 0;
  const int kind = kind_of(a, band_b);
  const dim3 g(grid);
  if (head_dim == 128) {
    BCP_LAUNCH_KIND(attn_bf16_narrow_kernel, 128, kNThreads)
  } else {
    BCP_LAUNCH_KIND(attn_bf16_narrow_kernel, 64, kNThreads)
  }
  return hipGetLastError();
}
#undef BCP_LAUNCH_KIND

}  // namespace bcp
