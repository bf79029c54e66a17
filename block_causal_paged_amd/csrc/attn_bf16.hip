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
// Work decomposition. A workgroup of 4 waves takes one work item: one kv head g, one
// q-tile of a sequence (tile_q positions x the G query heads of g = 256 packed rows,
// rho = position * G + head), and a contiguous chunk of that q-tile's non-skipped key
// tiles. Each wave owns 64 packed rows as two 32-column MFMA blocks.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, wave64). Scores are computed
// transposed, S^T = K Q^T: K rows are the A operand, queries the B operand, so each lane
// owns one query column and 16 key rows of every 32x32 block. The row max and row sum of
// the softmax are then in-lane reductions plus one exchange with lane^32. The output is
// also accumulated transposed, O^T += V^T P^T, with P^T taken straight from the score
// registers: the 8 keys a lane half contributes to one PV step are exactly the 8 score
// values it already holds, which fixes a permutation of the keys inside every 16-key
// group (bits 2 and 3 of the key index swapped). V stays row-major in LDS; gfx950's LDS
// transpose read (ds_read_b64_tr_b16) hands each lane 4 keys of one d column, and two of
// them per step deliver exactly those 8 keys as the A operand.
//
// Staging. Key and value tiles move HBM -> LDS with direct loads (global_load_lds_dwordx4),
// without passing through registers: the row addresses come from the page table two tiles
// ahead, the data one tile ahead (double-buffered LDS), so no load is waited on right after
// it is issued.
#include "bcp_internal.h"

namespace bcp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr float kLn2 = 0.69314718055994531f;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// LDS tiles. Key and value tiles are row-major [64 keys][d] with no padding, so the
// direct global->LDS loads (one 1 KB contiguous run per wave instruction) fill them; the
// 16-byte chunks of each row are XOR-swizzled instead (KSWZ, VSWZ below) so that the
// operand reads of the MFMA steps hit distinct LDS banks.
template <int HD>
struct AttnSmem {
  uint16_t q[kRowsPerWG][HD + 8];  // the work item's 256 packed query rows (B operand of S^T)
  uint16_t k[2][kTileK * HD];      // key tile, double buffered
  uint16_t v[2][kTileK * HD];      // value tile, double buffered
  int kblk[2][kTileK];             // block id of each key of a partial tile
};

// Chunk swizzles. K operand reads: 16 lanes read rows r..r+15 at one logical chunk, so
// the swizzle spreads consecutive rows over all 16-byte bank groups. V transpose reads:
// 32 lanes read 4 consecutive rows x 8 bytes x 8, so the swizzle moves each of the 4 rows
// to its own 64-byte window.
template <int HD>
__device__ __forceinline__ int kswz(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int HD>
__device__ __forceinline__ int vswz(int r) { return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }

struct Item {
  int s, g, q0, q_len, kvl;
};

// Rows of a key tile that one thread moves with direct global->LDS loads: wave w's
// instruction j covers LDS bytes [(w*NI + j) KB, +1 KB), i.e. RPI rows, and lane i copies
// 16 bytes of row (w*NI + j)*RPI + i/CPR at physical chunk i%CPR.
template <int HD>
struct DmaShape {
  static constexpr int CPR = HD / 8;          // 16-byte chunks per row
  static constexpr int RPI = 1024 / (2 * HD); // rows per 1 KB wave instruction
  static constexpr int NI = kTileK / RPI / 4; // instructions per wave per matrix
};

// Direct global->LDS copies, written as inline assembly so the compiler does not attach
// its conservative wait (it cannot tell the buffer being filled from the one being read);
// the kernel waits for them itself (wait_dma) right before the barrier that publishes the
// tile. Lane i of the wave writes LDS bytes [lds + size*i, +size).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// `lds` must be wave-uniform (it is, by construction, at every call).
__device__ __forceinline__ void dma16(const void* g, unsigned lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(base), "v"(g) : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Staging state of one key tile. Stage 1 (lookup) reads the plan entry and the physical
// pages: with page_size a multiple of 16 every 16-row group of a tile lies in one page, so
// the 4 group pages are wave-uniform scalar loads; other page sizes read one page id per
// lane and row. Stage 2 (fetch) issues the direct loads of K, V and (partial mode-B tiles)
// the key block ids. The main loop keeps one tile in each stage.
template <int NI>
struct Stage {
  int e;              // plan entry: (tile << 1) | is_partial; -1 when there is no tile
  int pg[4];          // page of each 16-row group (uniform), scalar-page path
  int row[NI];        // raw page id per staged row, per-lane path
};

template <int HD, int NI>
__device__ __forceinline__ void stage_lookup(const AttnArgs& a, const Item& it, int e, Stage<NI>& st) {
  using D = DmaShape<HD>;
  st.e = e;
  if (e < 0) return;
  const int vt = e >> 1;
  if (vt >= a.nct) return;                        // live tile: rows follow from the index
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (a.page_size % 16 == 0) {
    cint32* pt = as_const(a.page_table) + (int64_t)it.s * a.max_pages;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int lp, slot;
      page_split(vt * kTileK + 16 * q, a.page_size, a.page_shift, &lp, &slot);
      st.pg[q] = pt[min(lp, a.max_pages - 1)];
    }
  } else {
    const int32_t* pt = a.page_table + (int64_t)it.s * a.max_pages;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int j = vt * kTileK + (wave * NI + k) * D::RPI + lane / D::CPR;
      int lp, slot;
      page_split(j, a.page_size, a.page_shift, &lp, &slot);
      st.row[k] = pt[min(lp, a.max_pages - 1)];
    }
  }
}

// Number of keys of tile vt that exist (the rest of a partial tile is masked).
__device__ __forceinline__ int tile_valid(const AttnArgs& a, const Item& it, int vt) {
  return vt < a.nct ? clampi(it.kvl - vt * kTileK, 0, kTileK) : clampi(it.q_len - (vt - a.nct) * kTileK, 0, kTileK);
}

// Issue the direct loads of a resolved tile into LDS buffer `buf`. An absent key (past its
// region's length, or in a page outside the pool) copies the sequence's first live row:
// absent keys only occur in partial tiles, where the mask gives them weight exactly 0, and
// that row is finite, so it adds exactly nothing.
template <int HD, int NI>
__device__ __forceinline__ void stage_fetch(const AttnArgs& a, const Item& it, const Stage<NI>& st,
                                            AttnSmem<HD>& sm, int buf) {
  using D = DmaShape<HD>;
  const int vt = st.e >> 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool cached = vt < a.nct;
  const int nvalid = tile_valid(a, it, vt);
  const uint16_t* kb = (const uint16_t*)(cached ? a.k_cache : a.k_new);
  const uint16_t* vb = (const uint16_t*)(cached ? a.v_cache : a.v_new);
  const int64_t sub = ((int64_t)it.q0 * a.Hkv + it.g) * HD;   // substitute row for absent keys
  const bool scalar_pages = a.page_size % 16 == 0;
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int r = (wave * NI + k) * D::RPI + lane / D::CPR;    // row inside the tile
    const int pch = lane % D::CPR;                              // physical chunk
    int64_t row = -1;
    if (r < nvalid) {
      if (cached) {
        const int p = scalar_pages ? st.pg[wave] : st.row[k];
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
    const int kc = pch ^ kswz<HD>(r), vc = pch ^ vswz<HD>(r);
    dma16(ksrc + 8 * kc, lds_addr(&sm.k[buf][(wave * NI + k) * D::RPI * HD]));
    dma16(vsrc + 8 * vc, lds_addr(&sm.v[buf][(wave * NI + k) * D::RPI * HD]));
  }
  // Block ids of a partial tile's keys (wave 0, one key per lane). Mode A needs no memory;
  // mode B copies them; keys past nvalid are masked separately.
  if ((st.e & 1) && wave == 0) {
    const int j = (cached ? vt : vt - a.nct) * kTileK + lane;
    if (!a.mode_b) {
      sm.kblk[buf][lane] = lane >= nvalid ? kNoKeyBlk : (cached ? kNegInfBlk : j / a.block_size);
    } else {
      const int32_t* src = a.q_blk + it.q0;                    // in bounds, used when absent
      if (lane < nvalid) {
        if (cached) {
          const int q = lane >> 4;
          const int p = scalar_pages ? (q == 0 ? st.pg[0] : q == 1 ? st.pg[1] : q == 2 ? st.pg[2] : st.pg[3])
                                     : -1;
          int lp, slot;
          page_split(j, a.page_size, a.page_shift, &lp, &slot);
          if (scalar_pages && p >= 0 && p < a.num_pages) src = a.kv_blk + (int64_t)p * a.page_size + slot;
        } else {
          src = a.q_blk + it.q0 + j;
        }
      }
      dma4(src, lds_addr(&sm.kblk[buf][0]));
    }
  }
}

template <int HD>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  using D = DmaShape<HD>;
  constexpr int NI = D::NI;
  constexpr int CH = HD / 8;        // 16-byte chunks per row
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
    cint32* list = plan + L.list + (int64_t)u * a.nkt;
    auto entry = [&](int o) { return o < oe ? (int)list[o] : -1; };

    // Block id of each owned query column; invalid (padding) rows see every present key.
    int qblk[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int rho = wave * 64 + qb * 32 + col;
      const int pos = i0 + rho / G;
      qblk[qb] = pos >= it.q_len ? kNoKeyBlk - 1 : (a.mode_b ? a.q_blk[it.q0 + pos] : pos / a.block_size);
    }

    f32x16 o[2][NDB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[qb][db] = f32x16{};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    int n_partial = 0;
    __syncthreads();   // the previous item's reads of LDS are finished
    // Query rows into LDS: the G heads of one position are contiguous in q, so packed rows
    // rho .. rho+G-1 are one contiguous G*d run.
    for (int idx = tid; idx < kRowsPerWG * CH; idx += 256) {
      const int rho = idx / CH, c = idx - (idx / CH) * CH;
      const int pos = i0 + rho / G, hh = rho - (rho / G) * G;
      u32x4 v = {0, 0, 0, 0};
      if (pos < it.q_len)
        v = *(const u32x4*)(qg + ((int64_t)(it.q0 + pos) * a.Hq + (int64_t)it.g * G + hh) * HD + 8 * c);
      *(u32x4*)&sm.q[rho][8 * c] = v;
    }

    // Pipeline: the tile being computed sits in LDS; the next one's direct loads are in
    // flight; the one after has its rows resolved; e_far is the plan entry after that.
    Stage<NI> nx, nn;
    int e_cur = entry(ob);
    stage_lookup<HD, NI>(a, it, e_cur, nx);
    if (e_cur >= 0) stage_fetch<HD, NI>(a, it, nx, sm, 0);
    stage_lookup<HD, NI>(a, it, entry(ob + 1), nn);
    int e_far = entry(ob + 2);
    wait_dma();
    __syncthreads();

    for (int oi = ob; oi < oe; ++oi) {
      const int buf = (oi - ob) & 1;
      const bool partial = e_cur & 1;
      const int e_next = nn.e;
      nx = nn;
      if (e_next >= 0) stage_fetch<HD, NI>(a, it, nx, sm, buf ^ 1);
      stage_lookup<HD, NI>(a, it, e_far, nn);
      const int nvalid = tile_valid(a, it, e_cur >> 1);
      e_far = entry(oi + 3);
      n_partial += partial;
      const uint16_t* kt = sm.k[buf];
      const uint16_t* vt = sm.v[buf];

      // S^T = K Q^T for two 32-key blocks x two 32-query blocks.
      f32x16 sc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int krow = 32 * kb + col;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 kf = *(const bf16x8*)&kt[krow * HD + 8 * ((2 * t + hl) ^ kswz<HD>(krow))];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const bf16x8 qf = *(const bf16x8*)&sm.q[wave * 64 + qb * 32 + col][16 * t + 8 * hl];
            sc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, t == 0 ? f32x16{} : sc[qb][kb], 0, 0, 0);
          }
        }
      }

      // Mask, only on partial tiles. Lane (col, hl) holds key 32kb + 8(v/4) + 4hl + v%4.
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const i32x4 kbw = *(const i32x4*)&sm.kblk[buf][32 * kb + 8 * v4 + 4 * hl];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (kbw[c] > qblk[qb] || 32 * kb + 8 * v4 + 4 * hl + c >= nvalid)
                  sc[qb][kb][4 * v4 + c] = -INFINITY;
          }
      }

      // Online softmax in the log2 domain; P rounded to bf16 as the B operand of O^T += V^T P^T.
      bf16x8 pf[2][2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[qb][kb][v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // Lazy rescale: the reference max m only moves when a row's max grows by more than
        // 2^8 (or on the row's first visible key). Numerator and denominator both use m, so
        // the result is the same; P <= 2^8 stays well inside bf16 range.
        const float mcand = mx * sl2;
        const bool grow = mcand > m[qb] + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          // Rows that do not grow keep alpha = 1 (their m may still be -inf: no visible key yet).
          const float alpha = grow ? __builtin_amdgcn_exp2f(m[qb] - mcand) : 1.f;   // 0 if m was -inf
          m[qb] = grow ? mcand : m[qb];
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
        }
        const float muse = m[qb] == -INFINITY ? 0.f : m[qb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[qb][kb][v], sl2, -muse));
            sc[qb][kb][v] = p;
            rs += p;
          }
        l[qb] += rs;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            f32x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sc[qb][kb][8 * hs + e];
            pf[qb][kb][hs] = to_bf16x8(x);
          }
      }

      // O^T += V^T P^T. Step (kb, hs) covers keys 32kb+16hs .. +15; lane half hl feeds the
      // keys 32kb+16hs + {4hl..4hl+3, 8+4hl..8+4hl+3} (its score registers), which two
      // transpose reads deliver as the A operand, for d = 32db + lane%32.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const int ra = 32 * kb + 16 * hs + vrow0, rb = ra + 8;
            const int dcol = 32 * db + vcol0;
            const int ca = ((dcol >> 3) ^ vswz<HD>(ra)) * 8 + (dcol & 7);
            const int cb = ((dcol >> 3) ^ vswz<HD>(rb)) * 8 + (dcol & 7);
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[ra * HD + ca]);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)&vt[rb * HD + cb]);
            typedef __attribute__((ext_vector_type(8))) short s16x8;
            const bf16x8 vf = __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][hs], o[qb][db], 0, 0, 0);
          }

      wait_dma();        // this wave's direct loads of the next tile have landed
      __syncthreads();
      e_cur = e_next;
    }

    // Epilogue. Lane (col, hl) of block (qb, db) holds d = 32db + 8(v/4) + 4hl + v%4.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lt = l[qb] + __shfl_xor(l[qb], 32);
      const int rho = wave * 64 + qb * 32 + col;
      const int i = rho / G, hh = rho - (rho / G) * G, pos = i0 + i;
      if (pos >= it.q_len) continue;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse2 = lt > 0.f ? m[qb] + __log2f(lt) : -INFINITY;
      const int64_t row = (int64_t)(it.q0 + pos) * a.Hq + (int64_t)it.g * G + hh;
      if (pslot < 0) {
        uint16_t* op = (uint16_t*)a.out + row * HD;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            f32x4 x = {o[qb][db][4 * v4] * inv, o[qb][db][4 * v4 + 1] * inv, o[qb][db][4 * v4 + 2] * inv,
                       o[qb][db][4 * v4 + 3] * inv};
            typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
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
            f32x4 x = {o[qb][db][4 * v4] * inv, o[qb][db][4 * v4 + 1] * inv, o[qb][db][4 * v4 + 2] * inv,
                       o[qb][db][4 * v4 + 3] * inv};
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
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bcp
