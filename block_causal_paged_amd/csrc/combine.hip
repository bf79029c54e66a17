// Merge of split-KV partial results.
//
// A q-tile whose key tiles were cut into several chunks has one partial result per chunk:
// the chunk's softmax-normalized output O_c and its log-sum-exp lse_c (log2 domain). The
// softmax over the union of the chunks is their lse-weighted mean:
//   M = max_c lse_c,  w_c = 2^(lse_c - M),  O = sum_c w_c O_c / sum_c w_c,
//   lse = M + log2(sum_c w_c).
// This is the same online-softmax identity the attention kernel applies tile by tile. For
// bf16 steps the attention kernels store O_c in fp16, each row multiplied by a power of two
// that keeps it in range, and the factor that undoes it beside the LSE.
#include "bcp_internal.h"

namespace bcp {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
constexpr float kLn2 = 0.69314718055994531f;

template <int HD, bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  constexpr int V4 = HD / 4;              // float4 per row
  constexpr int RPW = 256 / V4;           // rows per work item (one row per V4 threads)
  constexpr int NGRP = kRowsPerWG / RPW;  // row groups per (split unit, kv head)
  constexpr int MAXC = 8;                 // splits whose loads are issued together
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt, a.Hkv);
  cint32* plan = as_const(a.plan);
  const int tid = threadIdx.x, d4 = tid % V4, rr = tid / V4;
  // The loads of a work item form two rounds: its split record (with the work count), then
  // the sequence's live rows and every partial result at once; the partial addresses do not
  // depend on the live rows, and rows past the sequence's live rows are not stored.
  // Row groups per split: all NGRP for 256-row q-tiles, fewer for narrow ones.
  const int ngrp = min(NGRP, (a.tile_q * a.G + RPW - 1) / RPW);
  // The first split record and the header arrive in one round trip (the records sit at a
  // place that does not depend on the step's shape); the check follows.
  bool ok;
  {
    PlanShape h = plan_shape(plan);
    cint32* sp = plan + L.split + 4 * (int64_t)min((int)blockIdx.x / NGRP, kWGs - 1);   // the wide case's first
    int r0 = sp[0], r1 = sp[1], r2 = sp[2], r3 = sp[3], ns = plan[kHdrSplit];
    asm volatile("" : "+s"(r0), "+s"(r1), "+s"(r2), "+s"(r3), "+s"(ns), "+s"(h.w[0]), "+s"(h.w[1]), "+s"(h.w[2]),
                 "+s"(h.w[3]), "+s"(h.w[4]), "+s"(h.w[5]), "+s"(h.w[6]), "+s"(h.w[7]), "+s"(h.w[8]), "+s"(h.w[9]),
                 "+s"(h.w[10]), "+s"(h.w[11]));
    ok = plan_matches(h, a);
  }
  if (!ok) return;
  for (int w = blockIdx.x; w < kWGs * ngrp; w += gridDim.x) {
    const int grp = w % ngrp, e = w / ngrp;
    cint32* sp = plan + L.split + 4 * (int64_t)e;   // inside the kWGs split records
    const int u = sp[0], g = sp[1], ps0 = sp[2], n = sp[3];
    if (w >= plan[kHdrSplit] * ngrp) break;
    const int s = u / a.nqt, r = u - (u / a.nqt) * a.nqt;
    const int rho = grp * RPW + rr;
    // Partial row of one piece: fp32 for fp32 steps; for bf16 steps fp16 values times the
    // row's restoring factor.
    auto partial = [&](int64_t slot) -> f32x4 {
      const int64_t row = slot * kRowsPerWG + rho;
      if constexpr (BF16_OUT)
        return __builtin_convertvector(*(const f16x4*)(a.part_h + row * HD + 4 * d4), f32x4) * a.part_scale[row];
      else
        return *(const f32x4*)(a.part_o + row * HD + 4 * d4);
    };
    float lc[MAXC];
    f32x4 oc[MAXC];
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {   // only the pair's own slots (n is uniform)
      lc[k] = -INFINITY;
      oc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k < n) {
        const int64_t slot = ps0 + k;
        lc[k] = a.part_lse[slot * kRowsPerWG + rho];
        oc[k] = partial(slot);
      }
    }
    int q0, q_len;
    live_rows(a.cu_q, s, a.total_q, a.max_q_len, &q0, &q_len);
    const int pos = r * a.tile_q + rho / a.G, hh = rho - (rho / a.G) * a.G;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) M = fmaxf(M, lc[k]);   // absent slots hold -inf
    for (int c = MAXC; c < n; ++c) M = fmaxf(M, a.part_lse[(int64_t)(ps0 + c) * kRowsPerWG + rho]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < MAXC; ++k) {
        const float wc = k < n ? __builtin_amdgcn_exp2f(lc[k] - M) : 0.f;
        acc += wc * oc[k];
        wsum += wc;
      }
      for (int c = MAXC; c < n; ++c) {
        const int64_t slot = ps0 + c;
        const float wc = __builtin_amdgcn_exp2f(a.part_lse[slot * kRowsPerWG + rho] - M);
        acc += wc * partial(slot);
        wsum += wc;
      }
      acc *= 1.f / wsum;
    }
    if (pos >= q_len) continue;
    const int64_t row = (int64_t)(q0 + pos) * a.Hq + (int64_t)g * a.G + hh;
    if constexpr (BF16_OUT) {
      *(bf16x4*)((uint16_t*)a.out + row * HD + 4 * d4) = __builtin_convertvector(acc, bf16x4);
    } else {
      *(f32x4*)((float*)a.out + row * HD + 4 * d4) = acc;
    }
    if (d4 == 0 && a.lse) a.lse[row] = M == -INFINITY ? -INFINITY : (M + __log2f(wsum)) * kLn2;
  }
}

}  // namespace

hipError_t launch_combine(const AttnArgs& a, int head_dim, int is_bf16, int grid, hipStream_t stream) {
  if (head_dim == 128) {
    if (is_bf16) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((combine_kernel<128, false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (is_bf16) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((combine_kernel<64, false>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bcp
