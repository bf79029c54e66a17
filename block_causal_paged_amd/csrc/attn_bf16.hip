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
// Work decomposition. A workgroup of 8 waves takes one work item: one kv head g, one
// q-tile of a sequence (tile_q positions x the G query heads of g = 256 packed rows,
// rho = position * G + head), and a contiguous chunk of that q-tile's non-skipped key
// tiles. Wave w owns packed rows [32w, 32w+32), one 32-column MFMA block; two waves share
// each SIMD, so one wave's matrix instructions overlap the other's softmax.
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
// without passing through registers, into a 3-stage ring: the tile two ahead is in flight
// while one is computed; physical pages are resolved one tile before that with scalar
// loads of the page table (each wave's 8 rows of a tile lie in one page when the page size
// is a multiple of 8).
#include "bcp_internal.h"

namespace bcp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 3;
constexpr int kRowsPerWave = kTileK / kWaves;   // key rows each wave stages per tile

// LDS: key and value tiles are row-major [64 keys][d] with no padding, so one direct-load
// wave instruction (a contiguous 1 KB run) fills whole rows; the 16-byte chunks of each
// row are XOR-swizzled (kswz, vswz) so that the operand reads hit distinct banks.
constexpr int kWin = 256;   // plan entries (and their pages) staged in LDS at a time

template <int HD>
struct AttnSmem {
  uint16_t k[kStages][kTileK * HD];
  uint16_t v[kStages][kTileK * HD];
  int kblk[kStages][kTileK];       // block id of each key of a partial tile
  int win_e[kWin];                 // the item's plan entries, one window at a time
  int win_pg[kWin][kWaves];        // page of each 8-row group of those tiles (cached tiles)
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
// bytes [lds + size*i, +size). `lds` is wave-uniform at every call.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* g, unsigned lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(base), "v"(g) : "memory");
}
// Wait until at most N of this wave's vector-memory loads are outstanding (they complete
// in issue order, so everything issued before the last N has landed).
template <int N>
__device__ __forceinline__ void wait_vm() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }

struct Item {
  int s, g, q0, q_len, kvl;
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

// Staging state of one key tile for one wave. Lookup resolves the physical page of the
// wave's 8 rows: from the page ids staged in LDS with the item's plan window when the page
// size is a multiple of 8, one vector load per lane and row otherwise. (The loop issues no
// scalar memory loads: those share a wait counter with LDS reads and, returning out of
// order, would make every LDS operand wait as long as a page-table miss.)
template <int NI>
struct Stage {
  int e;              // plan entry: (tile << 1) | is_partial; -1 when there is no tile
  int pw;             // page of this wave's rows (scalar path)
  int row[NI];        // raw page id per staged row (per-lane path)
  int krow;           // raw page id of row 8*wave + lane, lanes < 8 (per-lane path, block ids)
};

// `e` is the entry at window position `wi` (-1: no tile).
template <int HD, int NI>
__device__ __forceinline__ void stage_lookup(const AttnArgs& a, const Item& it, int e, int wi,
                                             const AttnSmem<HD>& sm, Stage<NI>& st) {
  using D = DmaShape<HD>;
  st.e = e;
  if (e < 0) return;
  const int vt = e >> 1;
  if (vt >= a.nct) return;                        // live tile: rows follow from the index
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (a.page_size % kRowsPerWave == 0) {
    st.pw = sm.win_pg[wi][wave];
  } else {
    const int32_t* pt = a.page_table + (int64_t)it.s * a.max_pages;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int j = vt * kTileK + kRowsPerWave * wave + k * D::RPI + lane / D::CPR;
      int lp, slot;
      page_split(j, a.page_size, a.page_shift, &lp, &slot);
      st.row[k] = pt[min(lp, a.max_pages - 1)];
    }
    if ((e & 1) && a.mode_b) {
      int lp, slot;
      page_split(vt * kTileK + kRowsPerWave * wave + (lane & 7), a.page_size, a.page_shift, &lp, &slot);
      st.krow = pt[min(lp, a.max_pages - 1)];
    }
  }
}

// Issue the direct loads of a resolved tile into LDS stage `sg`: NI K and NI V wave
// instructions per wave, plus one block-id copy on wave 0 for partial mode-B tiles. An
// absent key (past its region's length, or in a page outside the pool) copies the
// sequence's first live row: absent keys only occur in partial tiles, where the mask
// gives them weight exactly 0, and that row is finite, so it adds exactly nothing.
template <int HD, int NI>
__device__ __forceinline__ void stage_fetch(const AttnArgs& a, const Item& it, const Stage<NI>& st,
                                            AttnSmem<HD>& sm, int sg) {
  using D = DmaShape<HD>;
  const int vt = st.e >> 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool cached = vt < a.nct;
  const int nvalid = tile_valid(a, it, vt);
  const uint16_t* kb = (const uint16_t*)(cached ? a.k_cache : a.k_new);
  const uint16_t* vb = (const uint16_t*)(cached ? a.v_cache : a.v_new);
  const int64_t sub = ((int64_t)it.q0 * a.Hkv + it.g) * HD;   // substitute row for absent keys
  const bool scalar_pages = a.page_size % kRowsPerWave == 0;
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int r = kRowsPerWave * wave + k * D::RPI + lane / D::CPR;   // row inside the tile
    const int pch = lane % D::CPR;                                     // physical chunk
    int64_t row = -1;
    if (r < nvalid) {
      if (cached) {
        const int p = scalar_pages ? st.pw : st.row[k];
        if (p >= 0 && p < a.num_pages) {
          int lp, slot;
          page_split(vt * kTileK + r, a.page_size, a.page_shift, &lp, &slot);
          row = (int64_t)p * a.page_size + slot;
        }
      } else {
        row = it.q0 + (vt - a.nct) * kTileK + r;
      }
    }
    const bool ok = row >= 0;
    const uint16_t* ksrc = ok ? kb + (row * a.Hkv + it.g) * HD : (const uint16_t*)a.k_new + sub;
    const uint16_t* vsrc = ok ? vb + (row * a.Hkv + it.g) * HD : (const uint16_t*)a.v_new + sub;
    const int base = (kRowsPerWave * wave + k * D::RPI) * HD;
    dma16(ksrc + 8 * (pch ^ kswz<HD>(r)), lds_addr(&sm.k[sg][base]));
    dma16(vsrc + 8 * (pch ^ vswz<HD>(r)), lds_addr(&sm.v[sg][base]));
  }
  // Block ids of a partial tile's keys: each wave handles its own 8 rows (lanes 0..7).
  // Mode A needs no memory; mode B copies them with an exec-masked 4-byte direct load
  // (inactive lanes issue no request); keys past nvalid are masked separately.
  if (st.e & 1) {
    const int r = kRowsPerWave * wave + (lane & 7);
    const int j = (cached ? vt : vt - a.nct) * kTileK + r;
    if (!a.mode_b) {
      if (lane < 8) sm.kblk[sg][r] = r >= nvalid ? kNoKeyBlk : (cached ? kNegInfBlk : j / a.block_size);
    } else {
      const int32_t* src = a.q_blk + it.q0;                    // in bounds, used when absent
      if (r < nvalid) {
        if (cached) {
          int lp, slot;
          page_split(j, a.page_size, a.page_shift, &lp, &slot);
          const int p = scalar_pages ? st.pw : st.krow;
          if (p >= 0 && p < a.num_pages) src = a.kv_blk + (int64_t)p * a.page_size + slot;
        } else {
          src = a.q_blk + it.q0 + j;
        }
      }
      if (lane < 8) dma4(src, lds_addr(&sm.kblk[sg][kRowsPerWave * wave]));
    }
  }
}

// Publish a tile: this wave's loads of it have landed once at most the loads issued after
// it (the next tile's: 2*NI, plus the block-id copy of a partial mode-B tile) are
// outstanding; then the workgroup barrier makes every wave's share visible.
template <int HD>
__device__ __forceinline__ void land_tile(bool next_in_flight, bool next_extra) {
  constexpr int per = 2 * DmaShape<HD>::NI;
  if (!next_in_flight) wait_vm<0>();
  else if (next_extra) wait_vm<per + 1>();
  else wait_vm<per>();
  __syncthreads();
}

template <int HD>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnArgs a) {
  using D = DmaShape<HD>;
  constexpr int NI = D::NI;
  constexpr int NT = HD / 16;       // MFMA steps over d for the scores
  constexpr int NDB = HD / 32;      // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) AttnSmem<HD> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hl = lane >> 5;
  const int G = a.G;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt);
  cint32* plan = as_const(a.plan);
  const int n_work = plan[0] * a.Hkv;
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
  if (a.stats && blockIdx.x == 0 && tid == 0)   // skipped tiles of the whole grid, per kv head
    atomicAdd(&a.stats[2], (unsigned long long)a.Hkv * ((unsigned long long)L.units * a.nkt - plan[3]));

  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int item = w / a.Hkv;
    Item it;
    it.g = w - item * a.Hkv;
    cint32* ip = plan + L.items + 4 * (int64_t)item;
    const int u = ip[0], ob = ip[1], oe = ip[2], pslot = ip[3];
    it.s = u / a.nqt;
    const int r = u - it.s * a.nqt;
    live_rows(a.cu_q, it.s, a.total_q, a.max_q_len, &it.q0, &it.q_len);
    it.kvl = clampi(a.kv_len[it.s], 0, a.max_pages * a.page_size);
    const int i0 = r * a.tile_q;
    const int32_t* list = a.plan + L.list + (int64_t)u * a.nkt;

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

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float m = -INFINITY, l = 0.f;
    int n_partial = 0;

    // The item's tiles are processed in windows of kWin plan entries: the window's entries
    // and, for cached tiles, the page of each 8-row group are staged in LDS first, so the
    // tile loop reads its metadata from LDS only.
    for (int wb = ob; wb < oe; wb += kWin) {
      const int we = min(oe, wb + kWin);
      __syncthreads();   // earlier readers of LDS (previous window or item) are finished
      for (int i = tid; i < we - wb; i += kThreads) {
        const int e = list[wb + i];
        sm.win_e[i] = e;
        const int vt = e >> 1;
        if (vt < a.nct && a.page_size % kRowsPerWave == 0) {
          const int32_t* pt = a.page_table + (int64_t)it.s * a.max_pages;
#pragma unroll
          for (int q = 0; q < kWaves; ++q) {
            int lp, slot;
            page_split(vt * kTileK + kRowsPerWave * q, a.page_size, a.page_shift, &lp, &slot);
            sm.win_pg[i][q] = pt[min(lp, a.max_pages - 1)];
          }
        }
      }
      __syncthreads();
      auto entry = [&](int o) { return o < we ? sm.win_e[o - wb] : -1; };

    // Pipeline prologue: tiles wb and wb+1 in flight, wb+2 resolved.
    Stage<NI> s1, s2;
    int e_cur = entry(wb);
    stage_lookup<HD, NI>(a, it, e_cur, 0, sm, s1);
    const int e1 = entry(wb + 1);
    stage_lookup<HD, NI>(a, it, e1, 1, sm, s2);
    if (e_cur >= 0) stage_fetch<HD, NI>(a, it, s1, sm, wb % kStages);
    const bool extra1 = (e1 >= 0) && (e1 & 1) && a.mode_b;   // block-id copy
    if (e1 >= 0) stage_fetch<HD, NI>(a, it, s2, sm, (wb + 1) % kStages);
    stage_lookup<HD, NI>(a, it, entry(wb + 2), 2, sm, s1);
    land_tile<HD>(e1 >= 0, extra1);

    for (int oi = wb; oi < we; ++oi) {
      const int sg = oi % kStages;
      const bool partial = e_cur & 1;
      const int e_next = entry(oi + 1);
      const int e_ahead = s1.e;                 // tile oi+2, rows resolved
      const bool extra = (e_ahead >= 0) && (e_ahead & 1) && a.mode_b;
      if (e_ahead >= 0) stage_fetch<HD, NI>(a, it, s1, sm, (oi + 2) % kStages);
      stage_lookup<HD, NI>(a, it, entry(oi + 3), oi + 3 - wb, sm, s1);   // tile oi+3
      n_partial += partial;
      const uint16_t* kt = sm.k[sg];
      const uint16_t* vt = sm.v[sg];
      const int nvalid = tile_valid(a, it, e_cur >> 1);

      // S^T = K Q^T: two 32-key blocks x this wave's 32 query columns.
      f32x16 sc[2];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {      // alternate the two accumulators
          const bf16x8 kf = *(const bf16x8*)&kt[koff[t] + 32 * kb * HD];
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], t == 0 ? f32x16{} : sc[kb], 0, 0, 0);
        }
      }

      // Mask, only on partial tiles. Lane (col, hl) holds key 32kb + 8(v/4) + 4hl + v%4.
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const int k0 = 32 * kb + 8 * v4 + 4 * hl;
            const i32x4 kbw = *(const i32x4*)&sm.kblk[sg][k0];
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (kbw[c] > qblk || k0 + c >= nvalid) sc[kb][4 * v4 + c] = -INFINITY;
          }
      }

      // Online softmax in the log2 domain, with a lazy reference max: m only moves when a
      // row's max grows by more than 2^8 (or on its first visible key). Numerator and
      // denominator both use m, so the result is the same; P <= 2^8 fits bf16 easily.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mcand = mx * sl2;
      const bool grow = mcand > m + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        // Rows that do not grow keep alpha = 1 (their m may still be -inf).
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mcand) : 1.f;   // 0 if m was -inf
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
          for (int e = 0; e < 8; ++e) {
            x[e] = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * hs + e], sl2, -muse));
            rs += x[e];
          }
          pf[kb][hs] = to_bf16x8(x);
        }
      l += rs;

      // O^T += V^T P^T. Step (kb, hs) covers keys 32kb+16hs .. +15; lane half hl feeds the
      // keys 32kb+16hs + {4hl..4hl+3, 8+4hl..8+4hl+3} (its score registers), which two
      // transpose reads deliver as the A operand, for d = 32db + lane%32.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {    // consecutive steps use independent accumulators
            const int rofs = (32 * kb + 16 * hs) * HD;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[voff[db] + rofs]);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[voff[db] + rofs + 8 * HD]);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][hs], o[db], 0, 0, 0);
          }

      // Tile oi+1 must have landed (for every wave) before the next iteration reads it;
      // tile oi+2's loads may stay in flight.
      land_tile<HD>(e_ahead >= 0, extra);
      e_cur = e_next;
    }
    }   // window

    // Epilogue. Lane (col, hl) of block db holds d = 32db + 8(v/4) + 4hl + v%4.
    const float lt = l + __shfl_xor(l, 32);
    if (qvalid) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse2 = lt > 0.f ? m + __log2f(lt) : -INFINITY;
      const int64_t row = (int64_t)(it.q0 + pos) * a.Hq + (int64_t)it.g * G + hh;
      if (pslot < 0) {
        uint16_t* op = (uint16_t*)a.out + row * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            f32x4 x = {o[db][4 * v4] * inv, o[db][4 * v4 + 1] * inv, o[db][4 * v4 + 2] * inv, o[db][4 * v4 + 3] * inv};
            *(bf16x4*)(op + 32 * db + 8 * v4 + 4 * hl) = __builtin_convertvector(x, bf16x4);
          }
        if (hl == 0 && a.lse) a.lse[row] = lse2 * kLn2;
      } else {
        const int64_t slot = (int64_t)pslot * a.Hkv + it.g;
        float* pp = a.part_o + (slot * kRowsPerWG + rho) * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            f32x4 x = {o[db][4 * v4] * inv, o[db][4 * v4 + 1] * inv, o[db][4 * v4 + 2] * inv, o[db][4 * v4 + 3] * inv};
            *(f32x4*)(pp + 32 * db + 8 * v4 + 4 * hl) = x;
          }
        if (hl == 0) a.part_lse[slot * kRowsPerWG + rho] = lse2;
      }
    }

    if (a.stats && tid == 0) {
      const int n = oe - ob;
      atomicAdd(&a.stats[0], (unsigned long long)(n - n_partial));
      atomicAdd(&a.stats[1], (unsigned long long)n_partial);
      atomicAdd(&a.stats[3], (unsigned long long)n * 2ull * kTileK * HD * 2ull);
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bcp
