// Block-causal paged attention for float32 inputs, on the vector ALUs.
//
// Same definition, plan, tiling and online softmax as the bf16 matrix-core kernel, with
// every product and sum in float32 (gfx950's fp32 matrix rate equals its vector rate, so
// the simple formulation costs nothing in peak). Key and value tiles are staged in LDS and
// read by broadcast. A thread owns one packed query row (rho = position * G + head) of the
// workgroup's 256, or, when the item has at most 64 live rows, a quarter of one: the four
// threads of a row split each tile's keys and merge their softmax states at the end.
#include "bcp_internal.h"

namespace bcp {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr float kLn2 = 0.69314718055994531f;

template <int HD>
struct F32Smem {
  float ks[kTileK][HD];
  float vs[kTileK][HD];
  int kblk[kTileK];
  int kpos[kTileK];   // positions of a partial tile's keys (mode B with a window)
};

// One work item. SPLIT adjacent threads share a packed row: thread t takes row t / SPLIT and
// keys KS * (t % SPLIT) .. KS * (t % SPLIT + 1) - 1 of every tile (KS = kTileK / SPLIT), with
// its own online-softmax state; the SPLIT states of a row are merged at the end by the
// identity the combine kernel applies to split pieces (weights 2^(m_i - max m)). SPLIT = 4
// serves items with at most 64 live rows, whose one busy wave would otherwise walk every key
// of every tile alone. Returns the item's partial-tile count.
template <int HD, int SPLIT>
__device__ int f32_item(const AttnArgs& a, F32Smem<HD>& sm, int s, int g, int q0, int q_len, int kvl, int i0,
                        const int* list, int ob, int oe, int pslot) {
  constexpr int V4 = HD / 4;
  constexpr int KS = kTileK / SPLIT;
  const int tid = threadIdx.x;
  const int G = a.G;
  const float* qg = (const float*)a.q;
  const float sl2 = a.scale_log2;
  const int rho = tid / SPLIT, k0 = KS * (tid % SPLIT);
  const int pos = i0 + rho / G, hh = rho - (rho / G) * G;
  const bool valid = pos < q_len;
  const int64_t row = (int64_t)(q0 + pos) * a.Hq + (int64_t)g * G + hh;
  float qv[HD], ov[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qv[d] = valid ? qg[row * HD + d] : 0.f;
    ov[d] = 0.f;
  }
  const int qblk = !valid ? kNoKeyBlk - 1 : (a.mode_b ? a.q_blk[q0 + pos] : pos / a.block_size);
  const int qpos = valid && a.q_pos ? a.q_pos[q0 + pos] : 0;
  float m = -INFINITY, l = 0.f;
  int n_partial = 0;

  for (int oi = ob; oi < oe; ++oi) {
    const int e = list[oi];
    const int vt = e >> 1;
    const bool partial = e & 1;
    n_partial += partial;
    __syncthreads();
    for (int idx = tid; idx < kTileK * V4; idx += 256) {
      const int kappa = idx / V4, c = idx - (idx / V4) * V4;
      const float *kp = nullptr, *vp = nullptr;
      if (vt < a.nct) {
        const int j = vt * kTileK + kappa;
        const int p = j < kvl ? translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages) : -1;
        if (p >= 0) {
          const int64_t off = (((int64_t)p * a.page_size + (j % a.page_size)) * a.Hkv + g) * HD;
          kp = (const float*)a.k_cache + off;
          vp = (const float*)a.v_cache + off;
        }
      } else {
        const int j = (vt - a.nct) * kTileK + kappa;
        if (j < q_len && a.live_in_cache) {
          // Live row j read from the pool at logical row kv_len + j.
          const int p = translate_page(a.page_table, s, kvl + j, a.page_size, a.max_pages, a.num_pages);
          if (p >= 0) {
            const int64_t off = (((int64_t)p * a.page_size + ((kvl + j) % a.page_size)) * a.Hkv + g) * HD;
            kp = (const float*)a.k_cache + off;
            vp = (const float*)a.v_cache + off;
          }
        } else if (j < q_len) {
          const int64_t off = ((int64_t)(q0 + j) * a.Hkv + g) * HD;
          kp = (const float*)a.k_new + off;
          vp = (const float*)a.v_new + off;
        }
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)&sm.ks[kappa][4 * c] = kp ? *(const f32x4*)(kp + 4 * c) : z;
      *(f32x4*)&sm.vs[kappa][4 * c] = vp ? *(const f32x4*)(vp + 4 * c) : z;
    }
    if (partial && tid < kTileK) {
      int b, kp = 0;
      if (vt < a.nct) {
        const int j = vt * kTileK + tid;
        const int p = j < kvl ? translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages) : -1;
        b = p < 0 ? kNoKeyBlk : (a.mode_b ? a.kv_blk[(int64_t)p * a.page_size + (j % a.page_size)] : kNegInfBlk);
        if (p >= 0 && a.kv_pos) kp = a.kv_pos[(int64_t)p * a.page_size + (j % a.page_size)];
      } else {
        const int j = (vt - a.nct) * kTileK + tid;
        b = j >= q_len ? kNoKeyBlk : (a.mode_b ? a.q_blk[q0 + j] : j / a.block_size);
        if (j < q_len && a.q_pos) kp = a.q_pos[q0 + j];
      }
      sm.kblk[tid] = b;
      sm.kpos[tid] = kp;
    }
    __syncthreads();

    // Sliding window (mode A): key k of the tile lies wbase - k positions before this
    // row's query (committed row j at position j, live row i at kv_len + i).
    const int wbase = pos + (vt < a.nct ? kvl - vt * kTileK : -(vt - a.nct) * kTileK);
    const bool band = partial && a.window > 0 && !a.mode_b;
    const bool band_b = partial && a.window > 0 && a.mode_b;
    float sc[KS];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k = k0 + kk;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < HD; d += 4) {
        const f32x4 kv4 = *(const f32x4*)&sm.ks[k][d];
        acc = fmaf(qv[d], kv4[0], acc);
        acc = fmaf(qv[d + 1], kv4[1], acc);
        acc = fmaf(qv[d + 2], kv4[2], acc);
        acc = fmaf(qv[d + 3], kv4[3], acc);
      }
      if (partial && sm.kblk[k] > qblk) acc = -INFINITY;
      if (band && wbase - k >= a.window) acc = -INFINITY;
      if (band_b && (int64_t)qpos - sm.kpos[k] >= a.window) acc = -INFINITY;
      sc[kk] = acc;
      mx = fmaxf(mx, acc);
    }
    const float mnew = fmaxf(m, mx * sl2);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - muse);
    m = mnew;
    float rs = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) ov[d] *= alpha;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[kk], sl2, -muse));
      rs += p;
#pragma unroll
      for (int d = 0; d < HD; d += 4) {
        const f32x4 vv = *(const f32x4*)&sm.vs[k0 + kk][d];
        ov[d] = fmaf(p, vv[0], ov[d]);
        ov[d + 1] = fmaf(p, vv[1], ov[d + 1]);
        ov[d + 2] = fmaf(p, vv[2], ov[d + 2]);
        ov[d + 3] = fmaf(p, vv[3], ov[d + 3]);
      }
    }
    l = l * alpha + rs;
  }

  // Merge the SPLIT key slices of the row (adjacent lanes): each is weighted by 2^(m_i - M).
  if constexpr (SPLIT > 1) {
    float M = m;
#pragma unroll
    for (int x = 1; x < SPLIT; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
    const float w = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
    l *= w;
#pragma unroll
    for (int x = 1; x < SPLIT; x <<= 1) l += __shfl_xor(l, x);
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      float v = ov[d] * w;
#pragma unroll
      for (int x = 1; x < SPLIT; x <<= 1) v += __shfl_xor(v, x);
      ov[d] = v;
    }
    m = M;
  }

  if (valid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m + __log2f(l) : -INFINITY;
    // Each of the row's SPLIT threads stores its share of the d values.
    constexpr int DS = HD / SPLIT;
    const int d0 = DS * (tid % SPLIT);
    float* op = pslot < 0 ? (float*)a.out + row * HD : a.part_o + ((int64_t)pslot * kRowsPerWG + rho) * HD;
#pragma unroll
    for (int d = 0; d < HD; d += 4)
      if (d >= d0 && d < d0 + DS) *(f32x4*)(op + d) = f32x4{ov[d] * inv, ov[d + 1] * inv, ov[d + 2] * inv, ov[d + 3] * inv};
    if (tid % SPLIT == 0) {
      if (pslot < 0) {
        if (a.lse) a.lse[row] = lse2 * kLn2;
      } else {
        a.part_lse[(int64_t)pslot * kRowsPerWG + rho] = lse2;
      }
    }
  }
  return n_partial;
}

template <int HD>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) F32Smem<HD> sm;
  const int tid = threadIdx.x;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt, a.Hkv);
  const int rg = range_of_wg(blockIdx.x);
  if (!plan_matches(as_const(a.plan), a)) return;
  const int w_begin = a.plan[L.wg + rg], w_end = a.plan[L.wg + rg + 1];
  if (a.stats && blockIdx.x == 0 && tid == 0)   // skipped tiles of the whole grid, per kv head
    atomicAdd(&a.stats[2], (unsigned long long)a.Hkv * ((unsigned long long)L.units * a.nkt - a.plan[3]));

  for (int item = w_begin; item < w_end; ++item) {
    PlanItem pi;
    read_item(as_const(a.plan) + L.items + kItemWords * (int64_t)item, &pi);
    const int u = pi.u, g = pi.g, ob = pi.ob, oe = pi.oe, pslot = pi.pslot;
    const int s = u / a.nqt, r = u - (u / a.nqt) * a.nqt;
    const int q0 = pi.q0, q_len = pi.q_len, kvl = pi.kvl;
    const int i0 = r * a.tile_q;
    const int* list = a.plan + L.list + (int64_t)u * a.nkt;
    // Live rows of the q-tile: rho = position * G + head for positions below q_len, a
    // prefix of the 256 (uniform across the workgroup).
    const int nv = max(0, min(a.tile_q, q_len - i0)) * a.G;
    const int n_partial = nv <= 64 ? f32_item<HD, 4>(a, sm, s, g, q0, q_len, kvl, i0, list, ob, oe, pslot)
                                   : f32_item<HD, 1>(a, sm, s, g, q0, q_len, kvl, i0, list, ob, oe, pslot);
    if (a.stats && tid == 0) {
      const int n = oe - ob;
      atomicAdd(&a.stats[0], (unsigned long long)(n - n_partial));
      atomicAdd(&a.stats[1], (unsigned long long)n_partial);
      atomicAdd(&a.stats[3], (unsigned long long)n * 2ull * kTileK * HD * 4ull);
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bcp
