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

// Exclusive prefix sum over the workgroup (blockDim.x a multiple of 64, at most 1024).
// Returns this thread's exclusive prefix; *total receives the workgroup sum.
__device__ int block_scan_excl(int v, int* lds16, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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

// Maximum of v over the workgroup (every thread gets it).
__device__ int block_max(int v, int* lds16) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  if (lane == 0) lds16[wave] = x;
  __syncthreads();
  int all = lds16[0];
  for (int w = 1; w < nw; ++w) all = max(all, lds16[w]);
  __syncthreads();
  return all;
}

__global__ __launch_bounds__(256) void classify_kernel(ClassifyArgs a) {
  __shared__ int red[2][4];
  __shared__ int scan_lds[16];
  const int s = blockIdx.x / a.grid_q, r = blockIdx.x - (blockIdx.x / a.grid_q) * a.grid_q;
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

  const int64_t list_base = (int64_t)u * a.nkt;
  PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt);
  int running = 0;
  for (int base = 0; has_tiles && base < a.nkt; base += blockDim.x) {
    const int t = base + tid;
    int cls = BCP_TILE_SKIP;
    if (t < a.nkt && nrows > 0) {
      int nvalid, kmin, kmax;
      if (t < a.nct) {
        const int lo = t * a.tile_k;
        nvalid = clampi(kvl - lo, 0, a.tile_k);
        if (!a.mode_b) {
          kmin = kmax = kNegInfBlk;
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

// One workgroup turns the per-unit tile counts into balanced (unit, chunk) work items.
__global__ __launch_bounds__(1024) void planner_kernel(PlanArgs a) {
  __shared__ int scan_lds[16];
  int* plan = a.plan;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt);
  const int units = L.units;
  const int tid = threadIdx.x;

  // Total non-skipped tiles.
  int part = 0;
  for (int u = tid; u < units; u += blockDim.x) part += plan[L.cnt + u];
  int total_tiles;
  block_scan_excl(part, scan_lds, &total_tiles);

  const long long work = (long long)total_tiles * a.num_kv_heads;
  int chunk = (int)((work + kTargetWGs - 1) / kTargetWGs);
  chunk = max(chunk, kMinChunk);
  // Rounding each unit up to whole chunks can leave slightly more than kTargetWGs work
  // items, and the few left over would run as a second round after everything else. Take
  // the smallest chunk length that keeps the item count within kTargetWGs when one exists
  // (the count only falls as the chunk grows, so a bisection finds it).
  {
    int mx = 0;
    for (int u = tid; u < units; u += blockDim.x) mx = max(mx, plan[L.cnt + u]);
    const int cmax = block_max(mx, scan_lds);
    auto fits = [&](int c) {
      int p = 0, tot;
      for (int u = tid; u < units; u += blockDim.x) p += (plan[L.cnt + u] + c - 1) / c;
      block_scan_excl(p, scan_lds, &tot);
      return (long long)tot * a.num_kv_heads <= kTargetWGs;
    };
    if (cmax > chunk && !fits(chunk) && fits(cmax)) {
      int lo = chunk, hi = cmax;   // fits(lo) is false, fits(hi) is true
      while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if (fits(mid)) hi = mid;
        else lo = mid;
      }
      chunk = hi;
    }
  }

  int item_carry = 0, slot_carry = 0, split_carry = 0;
  for (int base = 0; base < units; base += blockDim.x) {
    const int u = base + tid;
    const int cnt = u < units ? plan[L.cnt + u] : 0;
    const int nch = (cnt + chunk - 1) / chunk;
    const bool split = nch > 1;
    int t_items, t_slots, t_split;
    const int item0 = item_carry + block_scan_excl(nch, scan_lds, &t_items);
    const int slot0 = slot_carry + block_scan_excl(split ? nch : 0, scan_lds, &t_slots);
    const int sidx = split_carry + block_scan_excl(split ? 1 : 0, scan_lds, &t_split);
    if (u < units) {
      for (int k = 0; k < nch; ++k) {
        int* it = plan + L.items + 4 * (int64_t)(item0 + k);
        it[0] = u;
        it[1] = (int)(((long long)k * cnt) / nch);
        it[2] = (int)(((long long)(k + 1) * cnt) / nch);
        it[3] = split ? slot0 + k : -1;
      }
      if (split) {
        int* sp = plan + L.split + 4 * (int64_t)sidx;
        sp[0] = u;
        sp[1] = slot0;
        sp[2] = nch;
        sp[3] = 0;
      }
    }
    item_carry += t_items;
    slot_carry += t_slots;
    split_carry += t_split;
  }
  if (tid == 0) {
    plan[0] = item_carry;
    plan[1] = split_carry;
    plan[2] = chunk;
    plan[3] = total_tiles;
    plan[4] = a.tile_q;
    plan[5] = a.tile_k;
    plan[6] = a.nqt;
    plan[7] = a.nkt;
  }
}

}  // namespace

hipError_t launch_classify(const ClassifyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(classify_kernel, dim3(a.batch * a.grid_q), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_planner(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(planner_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bcp
