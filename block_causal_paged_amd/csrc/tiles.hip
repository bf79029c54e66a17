// Tile classification of the block-causal mask, page translation of the tile grid, and the
// split-KV plan of a step.
//
// "Inference for Interpretable Text-Diffusion Models", section "FlexAttention with Aligned
// Tiles": the attention pattern is cut into tiles that are fully included (no masking),
// fully excluded (no work) or partial. Classes follow from block-id ranges: with qmin/qmax
// the smallest/largest block id over a tile's valid query rows and kmin/kmax over its valid
// key columns, the tile is SKIP iff it has no valid row or column or kmin > qmax (every
// key comes after every query's block), FULL iff kmax <= qmin and all tile_k columns are
// valid (every key is visible to every query), PARTIAL otherwise. Section "Paged
// Attention": the page table remaps the logical tile grid onto physical pages.
#include "bcp_internal.h"

namespace bcp {

namespace {

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then each row's total is added to
// the rows after it (row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}
__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_scan_incl(x), 63); }
// Maximum over the wave's lanes of non-negative values (0 fills the shifted-in lanes).
__device__ __forceinline__ int wave_max_nonneg(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// Exclusive prefix sum over the workgroup (blockDim.x a multiple of 64, at most 1024).
// Returns this thread's exclusive prefix; *total receives the workgroup sum.
__device__ int block_scan_excl(int v, int* lds16, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int x = wave_scan_incl(v);
  if (lane == 63) lds16[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    int t = lds16[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Maximum over the workgroup of non-negative values (every thread gets it); lds holds one
// int per wave.
__device__ int block_max_nonneg(int v, int* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max_nonneg(v);
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  int m = lds[0];
  for (int w = 1; w < nw; ++w) m = max(m, lds[w]);
  __syncthreads();
  return m;
}

constexpr int kClsLdsTiles = kMaxBandKeyTiles;   // key tiles whose mode-B block-id ranges fit in LDS
constexpr int kClsLdsRows = 512;     // q-tile rows staged in LDS for the exact mode-B window classes
typedef __attribute__((ext_vector_type(4))) int i32x4;

// Classifies q-tile r of sequence s (one workgroup of 256 threads; every thread calls it).
__device__ void classify_unit(const ClassifyArgs& a, int s, int r) {
  __shared__ int red[2][4];
  __shared__ int scan_lds[16];
  const bool has_tiles = r < a.nqt;     // false only for the phys_page-only launch of an empty grid
  const int u = s * a.nqt + r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int q0, q_len;
  live_rows(a.cu_q, s, a.total_q, a.max_q_len, &q0, &q_len);
  const int kvl = clampi(a.kv_len[s], 0, a.max_pages * a.page_size);
  const int i0 = r * a.tile_q;
  const int i1 = min(i0 + a.tile_q, q_len);
  const int nrows = max(0, i1 - i0);

  // Block-id range of the q-tile's valid rows.
  int qmin = 0, qmax = -1;
  if (nrows > 0) {
    if (!a.mode_b) {
      qmin = i0 / a.block_size;
      qmax = (i1 - 1) / a.block_size;
    } else {
      int mn = INT32_MAX, mx = INT32_MIN;
      for (int i = i0 + tid; i < i1; i += blockDim.x) {
        int b = a.q_blk[q0 + i];
        mn = min(mn, b);
        mx = max(mx, b);
      }
      mn = wave_min(mn);
      mx = wave_max(mx);
      if (lane == 0) { red[0][wave] = mn; red[1][wave] = mx; }
      __syncthreads();
      qmin = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
      qmax = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    }
  }

  // Mode B: block-id range of every key tile, computed cooperatively (one wave per tile,
  // one lane per key) into LDS when the grid fits; each thread then classifies its tiles.
  __shared__ int s_kmin[kClsLdsTiles], s_kmax[kClsLdsTiles];
  // (With a window the classes come from the pass below instead.)
  const bool coop = a.mode_b && a.window == 0 && has_tiles && nrows > 0 && a.nkt <= kClsLdsTiles;
  if (coop) {
    for (int t = wave; t < a.nkt; t += blockDim.x / 64) {
      int mn = INT32_MAX, mx = INT32_MIN;
      const bool cached = t < a.nct;
      const int lo = (cached ? t : t - a.nct) * a.tile_k;
      const int nvalid = clampi((cached ? kvl : q_len) - lo, 0, a.tile_k);
      for (int j = lo + lane; j < lo + nvalid; j += 64) {
        int b;
        if (cached) {
          const int p = translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages);
          b = p < 0 ? kNoKeyBlk : a.kv_blk[(int64_t)p * a.page_size + (j % a.page_size)];
        } else {
          b = a.q_blk[q0 + j];
        }
        mn = min(mn, b);
        mx = max(mx, b);
      }
      mn = wave_min(mn);
      mx = wave_max(mx);
      if (lane == 0) {
        s_kmin[t] = mn;
        s_kmax[t] = mx;
      }
    }
    __syncthreads();
  }

  // Mode B with a sliding window: a key is visible to a row iff its block id is not later
  // and it lies fewer than W positions before the row. One wave per key tile, one lane per
  // key: the tile is SKIP when its block ids or its positions are out of every row's reach,
  // FULL when both are within every row's reach (these range tests are exact), and
  // otherwise it is classified from its pairs, every row of the q-tile (staged in LDS) in
  // turn. The host rejects grids with more than kClsLdsTiles key tiles here.
  __shared__ unsigned char s_cls[kClsLdsTiles];
  __shared__ __attribute__((aligned(16))) int s_q2[kClsLdsRows][2];   // (block id, position) per row
  const bool band_b = a.mode_b && a.window > 0 && has_tiles && nrows > 0;
  if (band_b) {
    int pmn = INT32_MAX, pmx = INT32_MIN;
    for (int i = tid; i < nrows; i += blockDim.x) {
      const int b = a.q_blk[q0 + i0 + i], p = a.q_pos[q0 + i0 + i];
      pmn = min(pmn, p);
      pmx = max(pmx, p);
      if (i < kClsLdsRows) {
        s_q2[i][0] = b;
        s_q2[i][1] = p;
      }
    }
    pmn = wave_min(pmn);
    pmx = wave_max(pmx);
    __syncthreads();
    if (lane == 0) { red[0][wave] = pmn; red[1][wave] = pmx; }
    __syncthreads();
    const int64_t qpmin = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
    const int64_t qpmax = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    for (int t = wave; t < a.nkt; t += blockDim.x / 64) {
      const bool cached = t < a.nct;
      const int lo = (cached ? t : t - a.nct) * a.tile_k;
      const int nvalid = clampi((cached ? kvl : q_len) - lo, 0, a.tile_k);
      int kb = kNoKeyBlk, kp = 0, cls = BCP_TILE_SKIP;
      int bmn = INT32_MAX, bmx = INT32_MIN, kpmn = INT32_MAX, kpmx = INT32_MIN;
      for (int jj = lane; jj < a.tile_k; jj += 64) {   // one key per lane when tile_k <= 64
        const int j = lo + jj;
        int b = kNoKeyBlk, p = 0;
        if (jj < nvalid) {
          if (cached) {
            const int pg = translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages);
            if (pg >= 0) {
              const int64_t slot = (int64_t)pg * a.page_size + (j % a.page_size);
              b = a.kv_blk[slot];
              p = a.kv_pos[slot];
            }
          } else {
            b = a.q_blk[q0 + j];
            p = a.q_pos[q0 + j];
          }
          bmn = min(bmn, b);
          bmx = max(bmx, b);
          if (b != kNoKeyBlk) {
            kpmn = min(kpmn, p);
            kpmx = max(kpmx, p);
          }
        }
        if (jj < 64) { kb = b; kp = p; }
      }
      bmn = wave_min(bmn);
      bmx = wave_max(bmx);
      kpmn = wave_min(kpmn);
      kpmx = wave_max(kpmx);
      if (nvalid == 0 || bmn > qmax || kpmn == INT32_MAX || qpmin - kpmx >= a.window) {
        cls = BCP_TILE_SKIP;
      } else if (bmx <= qmin && nvalid == a.tile_k && qpmax - kpmn < a.window) {
        cls = BCP_TILE_FULL;
      } else if (a.tile_k <= 64 && nrows <= kClsLdsRows) {
        // Pairs: any / all over this lane's key and every row (two rows per LDS read).
        int any = 0, all = lane < nvalid && kb != kNoKeyBlk;
        const int64_t reach = (int64_t)kp + a.window;   // visible iff qb >= kb and qp < reach
        int i = 0;
        for (; i + 1 < nrows; i += 2) {
          const i32x4 w = *(const i32x4*)&s_q2[i][0];
          const bool v0 = w[0] >= kb && w[1] < reach, v1 = w[2] >= kb && w[3] < reach;
          any |= v0 | v1;
          all &= v0 & v1;
        }
        if (i < nrows) {
          const bool v0 = s_q2[i][0] >= kb && s_q2[i][1] < reach;
          any |= v0;
          all &= v0;
        }
        any &= lane < nvalid;
        const bool tany = __builtin_amdgcn_ballot_w64(any) != 0;
        const bool tall = nvalid == a.tile_k && __builtin_amdgcn_ballot_w64(lane < nvalid && !all) == 0;
        cls = !tany ? BCP_TILE_SKIP : tall ? BCP_TILE_FULL : BCP_TILE_PARTIAL;
      } else {
        // Tiles wider than a wave or q-tiles longer than the staging: pairs from memory.
        int any = 0, all = 1;
        for (int jj = lane; jj < a.tile_k; jj += 64) {
          const int j = lo + jj;
          int b = kNoKeyBlk, p = 0;
          if (jj < nvalid) {
            if (cached) {
              const int pg = translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages);
              if (pg >= 0) {
                const int64_t slot = (int64_t)pg * a.page_size + (j % a.page_size);
                b = a.kv_blk[slot];
                p = a.kv_pos[slot];
              }
            } else {
              b = a.q_blk[q0 + j];
              p = a.q_pos[q0 + j];
            }
          }
          int key_any = 0, key_all = jj < nvalid && b != kNoKeyBlk;
          for (int r2 = 0; r2 < nrows; ++r2) {
            const bool v = b <= a.q_blk[q0 + i0 + r2] && (int64_t)a.q_pos[q0 + i0 + r2] - p < a.window;
            key_any |= v;
            key_all &= v;
          }
          any |= key_any & (jj < nvalid);
          if (jj < nvalid) all &= key_all;
        }
        const bool tany = __builtin_amdgcn_ballot_w64(any) != 0;
        const bool tall = nvalid == a.tile_k && __builtin_amdgcn_ballot_w64(!all) == 0;
        cls = !tany ? BCP_TILE_SKIP : tall ? BCP_TILE_FULL : BCP_TILE_PARTIAL;
      }
      if (lane == 0 && t < kClsLdsTiles) s_cls[t] = (unsigned char)cls;
    }
    __syncthreads();
  }

  const int64_t list_base = (int64_t)u * a.nkt;
  PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt, a.num_kv_heads);
  int running = 0;
  for (int base = 0; has_tiles && base < a.nkt; base += blockDim.x) {
    const int t = base + tid;
    int cls = BCP_TILE_SKIP;
    if (t < a.nkt && band_b) {
      cls = s_cls[t];
    } else if (t < a.nkt && nrows > 0) {
      int nvalid, kmin, kmax;
      if (t < a.nct) {
        const int lo = t * a.tile_k;
        nvalid = clampi(kvl - lo, 0, a.tile_k);
        if (!a.mode_b) {
          kmin = kmax = kNegInfBlk;
        } else if (coop) {
          kmin = s_kmin[t];
          kmax = s_kmax[t];
        } else {
          kmin = INT32_MAX;
          kmax = INT32_MIN;
          for (int j = lo; j < lo + nvalid; ++j) {
            int p = translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages);
            int b = p < 0 ? kNoKeyBlk : a.kv_blk[(int64_t)p * a.page_size + (j % a.page_size)];
            kmin = min(kmin, b);
            kmax = max(kmax, b);
          }
        }
      } else {
        const int lo = (t - a.nct) * a.tile_k;
        nvalid = clampi(q_len - lo, 0, a.tile_k);
        if (!a.mode_b) {
          kmin = lo / a.block_size;
          kmax = (lo + max(nvalid, 1) - 1) / a.block_size;
        } else if (coop) {
          kmin = s_kmin[t];
          kmax = s_kmax[t];
        } else {
          kmin = INT32_MAX;
          kmax = INT32_MIN;
          for (int j = lo; j < lo + nvalid; ++j) {
            int b = a.q_blk[q0 + j];
            kmin = min(kmin, b);
            kmax = max(kmax, b);
          }
        }
      }
      if (nvalid == 0 || kmin > qmax) cls = BCP_TILE_SKIP;
      else if (kmax <= qmin && nvalid == a.tile_k) cls = BCP_TILE_FULL;
      else cls = BCP_TILE_PARTIAL;
      if (!a.mode_b && a.window > 0 && cls != BCP_TILE_SKIP) {
        // Sliding window (mode A): query row i sits at position kvl + i, committed key j at
        // j and live key j at kvl + j; a key is in the band while the query is fewer than
        // W positions past it. Rows i0..i1-1 against keys lo..hi of the tile:
        const int lo = (t < a.nct ? t : t - a.nct) * a.tile_k, hi = lo + nvalid - 1;
        const int64_t d_near = (t < a.nct ? (int64_t)kvl : 0) + i0 - hi;       // smallest distance
        const int64_t d_far = (t < a.nct ? (int64_t)kvl : 0) + (i1 - 1) - lo;  // largest distance
        if (t < a.nct) {
          if (d_near >= a.window) cls = BCP_TILE_SKIP;
          else if (d_far >= a.window) cls = BCP_TILE_PARTIAL;
        } else {
          // Key j is seen by the rows of its own block onwards, up to row j + W - 1; over
          // the tile's keys these row sets join into one interval.
          const int first = (lo / a.block_size) * a.block_size;
          const int64_t last = (int64_t)hi + a.window - 1;
          if (max(i0, first) > min((int64_t)i1 - 1, last)) cls = BCP_TILE_SKIP;
          else if (d_far >= a.window) cls = BCP_TILE_PARTIAL;
        }
      }
    }
    if (t < a.nkt && a.tile_class) a.tile_class[list_base + t] = (uint8_t)cls;
    if (a.plan) {
      int total;
      int ex = block_scan_excl(cls != BCP_TILE_SKIP ? 1 : 0, scan_lds, &total);
      if (t < a.nkt && cls != BCP_TILE_SKIP)
        a.plan[L.list + list_base + running + ex] = (t << 1) | (cls == BCP_TILE_PARTIAL ? 1 : 0);
      running += total;
    }
  }
  if (has_tiles && a.plan && tid == 0) a.plan[L.cnt + u] = running;

  // The page table applied to the cached tile grid, written once per sequence.
  if (a.phys_page && r == 0) {
    const int n = a.phys_tiles * a.phys_per_tile;
    for (int idx = tid; idx < n; idx += blockDim.x) {
      const int t = idx / a.phys_per_tile, k = idx - t * a.phys_per_tile;
      const int row = t * a.tile_k + k * a.page_size;
      int p = -1;
      if (row < kvl) p = translate_page(a.page_table, s, row, a.page_size, a.max_pages, a.num_pages);
      a.phys_page[(int64_t)s * n + idx] = p;
    }
  }
}

__global__ __launch_bounds__(256) void classify_kernel(ClassifyArgs a) {
  classify_unit(a, blockIdx.x / a.grid_q, blockIdx.x % a.grid_q);
}

// Exclusive prefix sums of three values at once over a workgroup of kPlanThreads.
constexpr int kPlanThreads = 256;
constexpr int kPlanLdsUnits = 4096;
constexpr int kPlanLdsSeqs = 1024;   // sequences whose live rows and length are staged in LDS
// Start-up cost of a work item (its first loads and its epilogue) in key-tile visits, as
// the stream-K cut counts it: about 10 us against about 2 us per visit.
constexpr unsigned kItemCost = 5;
struct Int3 {
  int x, y, z;
};
__device__ Int3 block_scan3_excl(Int3 v, Int3* lds, Int3* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Int3 s = {wave_scan_incl(v.x), wave_scan_incl(v.y), wave_scan_incl(v.z)};
  if (lane == 63) lds[wave] = s;
  __syncthreads();
  Int3 before = {0, 0, 0}, all = {0, 0, 0};
#pragma unroll
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    const Int3 t = lds[w];
    if (w < wave) {
      before.x += t.x;
      before.y += t.y;
      before.z += t.z;
    }
    all.x += t.x;
    all.y += t.y;
    all.z += t.z;
  }
  __syncthreads();
  *total = all;
  return Int3{before.x + s.x - v.x, before.y + s.y - v.y, before.z + s.z - v.z};
}

// Classes of a mode-A unit's key tiles in closed form (rows i0..i1-1 of a sequence with ql
// live rows and kvl committed ones; `window` 0 for none). In each region the non-skipped
// tiles are a run: cached tiles [t_lo, nc), live tiles [l_lo, nl); the FULL ones among them
// are the cached tiles in [tf_lo, nfc) and the live tiles in [lf_lo, nfl). Without a window
// a committed key is seen by every live row, so cached tile t is non-skipped when it holds a
// key and FULL when it holds tile_k; live tile j is non-skipped when its first key's block is
// at most the last row's block qmax, FULL when its tile_k keys exist and lie in blocks no
// later than the first row's block qmin. The window (query row i at position kvl + i,
// committed key j at j, live key j at kvl + j; seen while fewer than W positions behind)
// removes the tiles whose last key lies W or more positions before row i0, and leaves FULL
// only the tiles whose first key is fewer than W positions before row i1 - 1.
struct ModeABounds {
  int t_lo, nc, tf_lo, nfc, l_lo, nl, lf_lo, nfl;
};
__device__ ModeABounds mode_a_bounds(const PlanArgs& a, int ql, int kvl, int i0, int i1) {
  ModeABounds b = {0, 0, 0, 0, 0, 0, 0, 0};
  if (i1 <= i0) return b;
  const int tk = a.tile_k, D = a.block_size, nlt = a.nkt - a.nct;
  b.nc = min((kvl + tk - 1) / tk, a.nct);
  b.nfc = min(kvl / tk, a.nct);
  const int64_t qmax = (i1 - 1) / D, qmin = i0 / D;
  const int reach = (int)min<int64_t>((qmax + 1) * D, ql);   // keys a row of the q-tile may see
  const int full = (int)min<int64_t>((qmin + 1) * D, ql);    // keys every row of it sees
  b.nl = min((reach + tk - 1) / tk, nlt);
  b.nfl = min(full / tk, b.nl);
  if (a.window > 0) {
    const int64_t W = a.window;
    // First tile whose last key (at most the region's last) is within W of row i0.
    auto first_in = [&](int64_t last_key, int64_t need) -> int {   // need: that key's least index
      if (last_key < need) return INT32_MAX;
      const int64_t x = need + 1 - tk;                                  // t*tk + tk - 1 >= need
      return x <= 0 ? 0 : (int)((x + tk - 1) / tk);
    };
    auto first_full = [&](int64_t x) -> int { return x < 0 ? 0 : (int)(x / tk) + 1; };   // t*tk > x
    b.t_lo = min(first_in(kvl - 1, (int64_t)kvl + i0 - W + 1), b.nc);
    b.tf_lo = first_full((int64_t)kvl + i1 - 1 - W);
    b.l_lo = min(first_in(ql - 1, (int64_t)i0 - W + 1), b.nl);
    b.lf_lo = first_full((int64_t)i1 - 1 - W);
  }
  return b;
}

// One workgroup turns the per-unit tile counts into the ranges of the step's visits and
// the items (whole or partial (unit, kv head) pairs) that make them up. Each thread takes
// a contiguous run of units, then of pairs, so one scan orders everything.
__device__ void plan_step(const PlanArgs& a) {
  __shared__ Int3 scan_lds[kPlanThreads / 64];
  __shared__ int wg_first[kWGs + 1];
  __shared__ int s_cnt[kPlanLdsUnits], s_upre[kPlanLdsUnits], s_nepre[kPlanLdsUnits];
  int* plan = a.plan;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt, a.num_kv_heads);
  const int units = L.units, hkv = a.num_kv_heads;
  const int tid = threadIdx.x;
  // Per-unit counts and their prefix sums live in LDS when they fit (else in the plan).
  // So are each sequence's live rows and committed length, which every item carries.
  __shared__ int s_seq[kPlanLdsSeqs][3];
  const bool in_lds = units <= kPlanLdsUnits;
  const bool seq_lds = a.batch <= kPlanLdsSeqs;
  if (in_lds && !a.fused)
    for (int u = tid; u < units; u += kPlanThreads) s_cnt[u] = plan[L.cnt + u];
  // At most 64 (unit, kv head) pairs: wave 0 plans alone (below) while the other waves write
  // a fused step's classes and page entries.
  const bool one_wave = units * hkv <= 64;
  // A fused step's page entries: the first batch of page-table loads is issued here, beside
  // the length loads, for every entry inside max_pages_per_seq; which of them lie below the
  // committed length is decided when they are stored. So the page entries cost no round
  // trip of their own after the lengths.
  constexpr int kB = 4;
  const int pe_t0 = one_wave ? 64 : 0, pe_nthr = kPlanThreads - pe_t0;
  int pe_first[kB];
  auto page_entry = [&](int idx, int* sq, int* row, int* lp) {
    const int ppt = a.phys_per_tile, per_seq = a.nct * ppt, P = a.page_size;
    *sq = idx / per_seq;
    const int e = idx - *sq * per_seq;
    if (a.tile_k % P == 0) {
      *row = e * P;
      *lp = e;
    } else {
      const int t = e / ppt, k = e - t * ppt;
      *row = t * a.tile_k + k * P;
      *lp = *row / P;
    }
  };
  if (a.fused && a.phys_page && tid >= pe_t0) {
    const int total = a.batch * a.nct * a.phys_per_tile;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int idx = b * pe_nthr + tid - pe_t0;
      pe_first[b] = -1;
      if (idx < total) {
        int sq, row, lp;
        page_entry(idx, &sq, &row, &lp);
        if (lp < a.max_pages) pe_first[b] = a.page_table[(int64_t)sq * a.max_pages + lp];
      }
    }
  }
  // The header's length hash: the wrapping sum of every sequence's hash.
  __shared__ unsigned s_hash;
  if (tid == 0) s_hash = 0u;
  __syncthreads();
  unsigned my_hash = 0u;
  for (int sq = tid; sq < a.batch; sq += kPlanThreads) {
    int q0, ql;
    live_rows(a.cu_q, sq, a.total_q, a.max_q_len, &q0, &ql);
    const int kvl = clampi(a.kv_len[sq], 0, a.kv_cap);
    my_hash += seq_len_hash(sq, q0, ql, kvl);
    if (seq_lds) {
      s_seq[sq][0] = q0;
      s_seq[sq][1] = ql;
      s_seq[sq][2] = kvl;
    }
  }
  atomicAdd(&s_hash, my_hash);
  __syncthreads();
  // Tile classes, plan list entries and page entries of a fused step (each unit's classes
  // from mode_a_bounds, one unit per wave), written by threads [t0, t0 + nthr) (nthr a
  // multiple of 64).
  auto fused_entries = [&](int t0, int nthr) {
    {
      const int me = tid - t0, wave = me >> 6, lane = me & 63;
      for (int u = wave; u < units; u += nthr / 64) {
        const int sq = u / a.nqt, i0 = (u - sq * a.nqt) * a.tile_q, ql = s_seq[sq][1];
        const ModeABounds b = mode_a_bounds(a, ql, s_seq[sq][2], i0, min(i0 + a.tile_q, ql));
        int* list = plan + L.list + (int64_t)u * a.nkt;
        for (int t = lane; t < a.nkt; t += 64) {
          const int j = t - a.nct;   // live tile ordinal (negative for cached tiles)
          const bool on = j < 0 ? t >= b.t_lo && t < b.nc : j >= b.l_lo && j < b.nl;
          const bool full = j < 0 ? t >= b.tf_lo && t < b.nfc : j >= b.lf_lo && j < b.nfl;
          const int cls = !on ? BCP_TILE_SKIP : full ? BCP_TILE_FULL : BCP_TILE_PARTIAL;
          if (a.tile_class) a.tile_class[(int64_t)u * a.nkt + t] = (uint8_t)cls;
          if (on) list[j < 0 ? t - b.t_lo : b.nc - b.t_lo + j - b.l_lo] = (t << 1) | (full ? 0 : 1);
        }
      }
    }
    if (a.phys_page) {
      // Entry (sq, t, k) is the page of row t*tile_k + k*page_size; when pages tile the key
      // tiles exactly that row is e*page_size for the entry's ordinal e inside its sequence.
      // The loads of a batch of entries are issued before any of their stores; the first
      // batch was loaded at the start (threads t0.. of this call are the ones that did).
      const int me = tid - t0;
      const int total = a.batch * a.nct * a.phys_per_tile;
      for (int base = 0; base < total; base += kB * nthr) {
        int pv[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const int idx = base + b * nthr + me;
          pv[b] = -1;
          if (idx < total) {
            int sq, row, lp;
            page_entry(idx, &sq, &row, &lp);
            if (base == 0) pv[b] = pe_first[b];
            else if (lp < a.max_pages) pv[b] = a.page_table[(int64_t)sq * a.max_pages + lp];
            if (row >= s_seq[sq][2]) pv[b] = -1;
          }
        }
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const int idx = base + b * nthr + me;
          if (idx < total) a.phys_page[idx] = pv[b] >= 0 && pv[b] < a.num_pages ? pv[b] : -1;
        }
      }
    }
  };
  if (a.fused) {
    // Mode A (the host picks this only for such steps of at most kFusedPlanElems classes and
    // page entries, with the sequences in LDS): each unit's classes follow from its lengths
    // (mode_a_bounds), and a tile's place in its unit's list from the same bounds, without a
    // scan.
    for (int u = tid; u < units; u += kPlanThreads) {
      const int sq = u / a.nqt, i0 = (u - sq * a.nqt) * a.tile_q, ql = s_seq[sq][1];
      const ModeABounds b = mode_a_bounds(a, ql, s_seq[sq][2], i0, min(i0 + a.tile_q, ql));
      const int cnt = (b.nc - b.t_lo) + (b.nl - b.l_lo);
      plan[L.cnt + u] = cnt;
      s_cnt[u] = cnt;
    }
    __syncthreads();
    if (!one_wave) {
      fused_entries(pe_t0, pe_nthr);
      __syncthreads();   // the counts (in the plan when they do not fit in LDS) are read below
    }
  }
  auto cnt_of = [&](int u) { return in_lds ? s_cnt[u] : plan[L.cnt + u]; };
  // Writes item `idx` (unit u, kv head g, ordinals [ob, oe), partial slot ps) with the
  // unit's live rows and committed length, which the attention kernel then reads with the
  // item instead of loading them; the item that opens range r is also copied into the
  // range's record.
  auto put_item = [&](int64_t idx, int u, int g, int ob, int oe, int ps, int opens) {
    const int sq = u / a.nqt;
    int q0, ql, kvl;
    if (seq_lds) {
      q0 = s_seq[sq][0];
      ql = s_seq[sq][1];
      kvl = s_seq[sq][2];
    } else {
      live_rows(a.cu_q, sq, a.total_q, a.max_q_len, &q0, &ql);
      kvl = clampi(a.kv_len[sq], 0, a.kv_cap);
    }
    const int w[kItemWords] = {u, g, ob, oe, ps, q0, ql, kvl};
    int* it = plan + L.items + kItemWords * idx;
#pragma unroll
    for (int i = 0; i < kItemWords; ++i) it[i] = w[i];
    if (opens >= 0) {
      int* rec = plan + L.rng + kRngWords * (int64_t)opens;
#pragma unroll
      for (int i = 0; i < kItemWords; ++i) rec[2 + i] = w[i];
      rec[10] = 0;
      rec[11] = 0;
    }
  };

  // Items k = 0..n-1 of a pair of cnt visits cut into n near-equal chunks: chunk k covers
  // ordinals [floor(k*cnt/n), floor((k+1)*cnt/n)), stepped without a division per item.
  auto put_chunks = [&](int first, int u, int g, int cnt, int n, int slot0) {
    const int q = n > 0 ? cnt / n : 0, rr = cnt - q * n;
    int ob = 0, acc = 0;
    for (int k = 0; k < n; ++k) {
      int oe = ob + q;
      acc += rr;
      if (acc >= n) {
        acc -= n;
        ++oe;
      }
      put_item(first + k, u, g, ob, oe, slot0 >= 0 ? slot0 + k : -1, first + k);
      wg_first[first + k] = first + k;
      ob = oe;
    }
  };
  // The chunk length search of the decode path below: among kCand candidate lengths
  // lo + step*(j+1) (capped at hi) it keeps the smallest whose chunk count fits in kWGs as
  // the new hi and the largest that does not as the new lo. count(j) is the chunk count at
  // candidate j summed over all pairs.
  constexpr int kCand = 8;
  auto narrow = [&](int& lo, int& hi, int step, auto count) {
    int new_lo = lo, new_hi = hi;
#pragma unroll
    for (int j = kCand - 1; j >= 0; --j) {
      const int cj = min(lo + step * (j + 1), hi);
      if (count(j) <= kWGs) new_hi = cj;   // the smallest fitting candidate wins
      else if (new_lo == lo) new_lo = cj;  // the largest failing candidate
    }
    lo = new_lo;   // chunk counts fall as the length grows, so new_lo < new_hi
    hi = new_hi;
  };
  // The header: item and split-pair counts, ranges, visits, tile sizes, then the words
  // that the kernels and the host compare with their own arguments.
  auto write_header = [&](int n_items, int n_split, unsigned n_ranges, int total_tiles) {
    plan[0] = n_items;
    plan[1] = n_split;
    plan[2] = n_ranges;
    plan[3] = total_tiles;
    plan[4] = a.tile_q;
    plan[5] = a.tile_k;
    plan[6] = a.nqt;
    plan[7] = a.nkt;
    plan[kHdrMagic] = kPlanMagic;
    plan[kHdrBatch] = a.batch;
    plan[kHdrHkv] = a.num_kv_heads;
    plan[kHdrLenHash] = (int)s_hash;
    plan[kHdrWindow] = a.window;
    plan[kHdrModeB] = a.mode_b;
    plan[kHdrTotalQ] = a.total_q;
    plan[kHdrKvCap] = a.kv_cap;
  };
  if (one_wave) {
    if (tid >= 64) {
      if (a.fused) fused_entries(pe_t0, pe_nthr);
      return;
    }
    // The decode path below with every unit and every pair on a lane of wave 0: its sums and
    // scans are wave operations, with no barrier.
    const int lane = tid;
    const int cu = lane < units ? cnt_of(lane) : 0;
    const int cu_incl = wave_scan_incl(cu);
    const int total_tiles = __builtin_amdgcn_readlane(cu_incl, 63);
    if (lane < units) plan[L.upre + lane] = cu_incl - cu;
    if (lane == 0) plan[L.upre + units] = total_tiles;
    const unsigned W = (unsigned)total_tiles * (unsigned)hkv;
    const int pairs = units * hkv;
    const int pr = lane;
    const int u = pr < pairs ? pr % units : 0, g = pr < pairs ? pr / units : 0;
    const int cnt = pr < pairs ? cnt_of(u) : 0;
    const int cmax = wave_max_nonneg(cnt);
    int c = max(kMinChunk, (int)((W + kWGs - 1) / kWGs));
    if (cmax > c) {
      int lo = c - 1, hi = cmax;
      bool first = true;
      while (hi - lo > 1) {
        const int step = first ? 1 : (hi - lo + kCand) / (kCand + 1);
        first = false;
        int sums[kCand];
#pragma unroll
        for (int j = 0; j < kCand; ++j) {
          const int cj = min(lo + step * (j + 1), hi);
          sums[j] = wave_sum((cnt + cj - 1) / cj);
        }
        narrow(lo, hi, step, [&](int j) { return sums[j]; });
      }
      c = hi;
    }
    const int n = cnt > 0 ? (cnt + c - 1) / c : 0;
    const bool split = n > 1;
    const int in = wave_scan_incl(n), isp = wave_scan_incl(split ? n : 0), ip = wave_scan_incl(split ? 1 : 0);
    const int n_items = __builtin_amdgcn_readlane(in, 63);
    put_chunks(in - n, u, g, cnt, n, split ? isp - n : -1);
    if (split) {
      int* sp = plan + L.split + 4 * (int64_t)(ip - 1);
      sp[0] = u;
      sp[1] = g;
      sp[2] = isp - n;
      sp[3] = n;
    }
    // Range r opens item r for every r below the item count and is empty after it, so its
    // first item is min(r, items) (the suffix minimum of the general path, in closed form).
    for (int w = lane; w <= kWGs; w += 64) {
      const int f = min(w, n_items);
      plan[L.wg + w] = f;
      if (w < kWGs) {
        plan[L.rng + kRngWords * (int64_t)w] = f;
        plan[L.rng + kRngWords * (int64_t)w + 1] = min(w + 1, n_items);
      }
    }
    if (lane == 0) write_header(n_items, __builtin_amdgcn_readlane(ip, 63), max(1, n_items), total_tiles);
    return;
  }

  // Prefix sums of the per-unit tile counts.
  const int upt = (units + kPlanThreads - 1) / kPlanThreads;
  const int u0 = min(units, tid * upt), u1 = min(units, u0 + upt);
  // (With them, the number of units with tiles before each unit.)
  int mine = 0, mine_ne = 0;
  for (int u = u0; u < u1; ++u) {
    mine += cnt_of(u);
    mine_ne += cnt_of(u) > 0;
  }
  Int3 tot;
  const Int3 run3 = block_scan3_excl(Int3{mine, mine_ne, 0}, scan_lds, &tot);
  int run = run3.x, run_ne = run3.y;
  for (int u = u0; u < u1; ++u) {
    plan[L.upre + u] = run;
    if (in_lds) {
      s_upre[u] = run;
      s_nepre[u] = run_ne;
    }
    run += cnt_of(u);
    run_ne += cnt_of(u) > 0;
  }
  const int total_tiles = tot.x;
  if (tid == 0) plan[L.upre + units] = total_tiles;
  for (int w = tid; w <= kWGs; w += kPlanThreads) wg_first[w] = INT32_MAX;
  __syncthreads();   // upre is read back below by other threads
  auto upre_of = [&](int u) { return in_lds ? s_upre[u] : plan[L.upre + u]; };

  const unsigned W = (unsigned)total_tiles * (unsigned)hkv;
  const int pairs = units * hkv;
  unsigned n_wg = 1;
  Int3 all = {0, 0, 0};

  if (pairs <= kPlanThreads) {
    // Few (unit, kv head) pairs (decode batches): cut each pair into ceil(cnt/c) near-equal
    // chunks, one range each, with the smallest chunk length c >= max(kMinChunk,
    // ceil(W/kWGs)) that keeps the chunk count within kWGs (the count only falls as c
    // grows, so a bisection finds it). One item per range, at most c visits long.
    const int pr = tid;
    const int u = pr < pairs ? pr % units : 0, g = pr < pairs ? pr / units : 0;
    const int cnt = pr < pairs ? cnt_of(u) : 0;
    // The search tests kCand chunk lengths per round: the chunk counts of all candidates
    // are summed over the pairs at once (wave sums, then one exchange through LDS). The
    // first round tries the kCand lengths from the lower bound up, which settles the usual
    // case; later rounds spread the candidates over the remaining interval, which shrinks
    // to the gap between the last length that gives too many chunks and the next one.
    __shared__ int cand_lds[kPlanThreads / 64][kCand];
    const int cmax = block_max_nonneg(cnt, (int*)scan_lds);
    int c = max(kMinChunk, (int)((W + kWGs - 1) / kWGs));
    if (cmax > c) {
      int lo = c - 1, hi = cmax;   // too many chunks at lo (or lo below the start); <= kWGs at hi
      bool first = true;
      while (hi - lo > 1) {
        const int step = first ? 1 : (hi - lo + kCand) / (kCand + 1);   // lo + step*(j+1)
        first = false;
        const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int j = 0; j < kCand; ++j) {
          const int cj = min(lo + step * (j + 1), hi);
          const int nj = wave_sum((cnt + cj - 1) / cj);
          if (lane == 0) cand_lds[wave][j] = nj;
        }
        __syncthreads();
        narrow(lo, hi, step, [&](int j) {
          int tot = 0;
#pragma unroll
          for (int w = 0; w < kPlanThreads / 64; ++w) tot += cand_lds[w][j];
          return tot;
        });
        __syncthreads();
      }
      c = hi;
    }
    const int n = cnt > 0 ? (cnt + c - 1) / c : 0;
    const bool split = n > 1;
    const Int3 at = block_scan3_excl(Int3{n, split ? n : 0, split ? 1 : 0}, scan_lds, &all);
    put_chunks(at.x, u, g, cnt, n, split ? at.y : -1);
    if (split) {
      int* sp = plan + L.split + 4 * (int64_t)at.z;
      sp[0] = u;
      sp[1] = g;
      sp[2] = at.y;
      sp[3] = n;
    }
    n_wg = max(1, all.x);
  } else {
    // The pairs, head-major, are laid end to end in a virtual sequence in which each pair
    // with tiles is its kItemCost start-up positions (standing for the work item's fixed
    // cost: its first loads and its epilogue) followed by its visits. Range r covers
    // positions [b(r), b(r+1)) of the Wv positions, for n_wg <= kWGs ranges: the first `rem`
    // ranges have q + 1 positions, the others q. So a range that starts more items gets
    // fewer visits. (32-bit: the plan supports steps of fewer than 2^31 positions.)
    const unsigned C = in_lds ? kItemCost : 0, NE = (unsigned)tot.y;
    const unsigned Wv = W + C * (unsigned)hkv * NE;
    n_wg = max(1u, min((unsigned)kWGs, Wv / kMinChunk));
    const unsigned q = Wv / n_wg, rem = Wv - q * n_wg, big = rem * (q + 1);
    auto b = [&](unsigned r) { return r * q + min(r, rem); };
    auto range_of = [&](unsigned x) { return x < big ? x / (q + 1) : rem + (x - big) / q; };
    // Pair pr = (kv head g, unit u): its start-up positions begin at
    // Sv = g*(T + C*NE) + upre[u] + C*nepre[u], its visits at S = Sv + C.
    auto pair_info = [&](int pr, int* u, int* g, int* cnt, unsigned* S, unsigned* rf, unsigned* Sv) {
      *g = pr / units;
      *u = pr - *g * units;
      *cnt = cnt_of(*u);
      *Sv = (unsigned)*g * ((unsigned)total_tiles + C * NE) + (unsigned)upre_of(*u) +
            (C ? C * (unsigned)s_nepre[*u] : 0u);
      *S = *Sv + C;
      *rf = *cnt > 0 ? range_of(*S) : 0;
      return *cnt > 0 ? (int)(range_of(*S + *cnt - 1) - *rf) + 1 : 0;   // pieces
    };

    const int ppt = (pairs + kPlanThreads - 1) / kPlanThreads;
    const int p0 = min(pairs, tid * ppt), p1 = min(pairs, p0 + ppt);
    Int3 own = {0, 0, 0};   // items, partial slots, split pairs of this thread's pairs
    for (int pr = p0; pr < p1; ++pr) {
      int u, g, cnt;
      unsigned S, rf, Sv;
      const int n = pair_info(pr, &u, &g, &cnt, &S, &rf, &Sv);
      own.x += n;
      own.y += n > 1 ? n : 0;
      own.z += n > 1 ? 1 : 0;
    }
    Int3 at = block_scan3_excl(own, scan_lds, &all);
    for (int pr = p0; pr < p1; ++pr) {
      int u, g, cnt;
      unsigned S, rf, Sv;
      const int n = pair_info(pr, &u, &g, &cnt, &S, &rf, &Sv);
      const bool split = n > 1;
      for (int k = 0; k < n; ++k) {
        const unsigned r = rf + k;
        const unsigned lo = max(b(r), S), hi = min(b(r + 1), S + cnt);
        // The piece opens range r (is its first item) when no earlier pair's visits lie in
        // it: later pieces start at b(r); the first one when the pair's start-up positions
        // begin at or before b(r) (the previous pair's positions end where they begin).
        const bool opens = k > 0 || Sv <= b(r);
        put_item(at.x + k, u, g, (int)(lo - S), (int)(hi - S), split ? at.y + k : -1, opens ? (int)r : -1);
        if (opens) wg_first[r] = at.x + k;
      }
      if (split) {
        int* sp = plan + L.split + 4 * (int64_t)at.z;
        sp[0] = u;
        sp[1] = g;
        sp[2] = at.y;
        sp[3] = n;
      }
      at.x += n;
      at.y += split ? n : 0;
      at.z += split ? 1 : 0;
    }
  }
  if (tid == 0) wg_first[kWGs] = all.x;
  __syncthreads();
  // A range that opens no item (an empty one, or one past n_wg) starts where the next
  // range does: the suffix minimum over the opened starts (which increase with r).
  {
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int PER = (kWGs + 1 + kPlanThreads - 1) / kPlanThreads;   // entries per thread
    int v[PER];
    int m = INT32_MAX;
#pragma unroll
    for (int k = PER - 1; k >= 0; --k) {
      const int w = tid * PER + k;
      v[k] = w <= kWGs ? wg_first[w] : INT32_MAX;
      m = min(m, v[k]);
      v[k] = m;   // suffix min inside this thread's entries
    }
    // Suffix min across threads: min over the entries of later threads.
    int x = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_down(x, o);
      if (lane + o < 64) x = min(x, y);
    }
    __shared__ int wave_min[kPlanThreads / 64];
    if (lane == 0) wave_min[wave] = x;
    __syncthreads();
    int later = __shfl_down(x, 1);
    if (lane == 63) later = INT32_MAX;
    for (int w = wave + 1; w < kPlanThreads / 64; ++w) later = min(later, wave_min[w]);
    __syncthreads();   // every thread has read wg_first
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int w = tid * PER + k;
      if (w <= kWGs) {
        plan[L.wg + w] = min(v[k], later);
        wg_first[w] = min(v[k], later);
      }
    }
    __syncthreads();
    for (int w = tid; w < kWGs; w += kPlanThreads) {
      plan[L.rng + kRngWords * (int64_t)w] = wg_first[w];
      plan[L.rng + kRngWords * (int64_t)w + 1] = wg_first[w + 1];
    }
  }
  if (tid == 0) write_header(all.x, all.z, n_wg, total_tiles);
}

__global__ __launch_bounds__(kPlanThreads) void planner_kernel(PlanArgs a) { plan_step(a); }

}  // namespace

hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(classify_kernel, dim3(a.batch * a.grid_q), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_planner(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(planner_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bcp
