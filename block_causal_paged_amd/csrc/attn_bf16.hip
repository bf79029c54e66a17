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
// group (bits 2 and 3 of the key index swapped). V is staged into LDS transposed,
// [d][permuted key], so the A operand of the PV step is one 16-byte LDS read.
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

template <int HD>
struct AttnSmem {
  uint16_t q[kRowsPerWG][HD + 8];  // the work item's 256 packed query rows (B operand of S^T)
  uint16_t k[2][kTileK][HD + 8];   // key rows, padded so the A-operand reads hit distinct banks
  uint16_t vt[2][HD * kTileK];     // V transposed: [d][permuted key], 16-byte XOR swizzle
  int kblk[2][kTileK];             // block id of each key of a partial tile
};

// Position of key kappa in a transposed V row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int kappa) {
  return (kappa & ~12) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}
// Element offset of (d, pos) in a transposed V tile; 16-byte chunks XOR-swizzled by d.
__device__ __forceinline__ int vt_off(int d, int pos) {
  const int swz = ((d >> 1) ^ (d >> 3)) & 7;
  return d * kTileK + ((((pos >> 3) ^ swz)) << 3) + (pos & 7);
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }

struct Item {
  int s, g, q0, q_len, kvl;
};

// Device address of row `kappa` of virtual key tile `vt` for kv head g, or null when the key
// is absent (past the length, or in a page outside the pool).
template <int HD>
__device__ __forceinline__ const uint16_t* key_row(const AttnArgs& a, const uint16_t* cache,
                                                   const uint16_t* live, int vt, int kappa,
                                                   const Item& it) {
  if (vt < a.nct) {
    const int j = vt * kTileK + kappa;
    if (j >= it.kvl) return nullptr;
    const int p = translate_page(a.page_table, it.s, j, a.page_size, a.max_pages, a.num_pages);
    if (p < 0) return nullptr;
    return cache + (((int64_t)p * a.page_size + (j % a.page_size)) * a.Hkv + it.g) * HD;
  }
  const int j = (vt - a.nct) * kTileK + kappa;
  if (j >= it.q_len) return nullptr;
  return live + ((int64_t)(it.q0 + j) * a.Hkv + it.g) * HD;
}

// Block id of key kappa of tile vt for the mask: committed rows are -inf in mode A,
// absent keys +inf.
__device__ __forceinline__ int key_block(const AttnArgs& a, int vt, int kappa, const Item& it) {
  if (vt < a.nct) {
    const int j = vt * kTileK + kappa;
    if (j >= it.kvl) return kNoKeyBlk;
    const int p = translate_page(a.page_table, it.s, j, a.page_size, a.max_pages, a.num_pages);
    if (p < 0) return kNoKeyBlk;
    return a.mode_b ? a.kv_blk[(int64_t)p * a.page_size + (j % a.page_size)] : kNegInfBlk;
  }
  const int j = (vt - a.nct) * kTileK + kappa;
  if (j >= it.q_len) return kNoKeyBlk;
  return a.mode_b ? a.q_blk[it.q0 + j] : j / a.block_size;
}

template <int HD>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int CH = HD / 8;        // 16-byte chunks per key row
  constexpr int KPT = CH / 4;       // consecutive keys each thread stages per tile
  constexpr int NT = HD / 16;       // MFMA steps over d for the scores
  constexpr int NDB = HD / 32;      // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) AttnSmem<HD> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hl = lane >> 5;
  const int G = a.G;
  const PlanLayout L = plan_layout(a.batch, a.nqt, a.nkt);
  const int n_work = a.plan[0] * a.Hkv;
  const uint16_t* qg = (const uint16_t*)a.q;
  const uint16_t* kcache = (const uint16_t*)a.k_cache;
  const uint16_t* vcache = (const uint16_t*)a.v_cache;
  const uint16_t* knew = (const uint16_t*)a.k_new;
  const uint16_t* vnew = (const uint16_t*)a.v_new;
  const int st_kg = tid / CH, st_c = tid - (tid / CH) * CH;   // staging: key group, chunk
  const float sl2 = a.scale_log2;
  if (a.stats && blockIdx.x == 0 && tid == 0)   // skipped tiles of the whole grid, per kv head
    atomicAdd(&a.stats[2], (unsigned long long)a.Hkv * ((unsigned long long)L.units * a.nkt - a.plan[3]));

  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int item = w / a.Hkv;
    Item it;
    it.g = w - item * a.Hkv;
    const int* ip = a.plan + L.items + 4 * (int64_t)item;
    const int u = ip[0], ob = ip[1], oe = ip[2], pslot = ip[3];
    it.s = u / a.nqt;
    const int r = u - it.s * a.nqt;
    live_rows(a.cu_q, it.s, a.total_q, a.max_q_len, &it.q0, &it.q_len);
    it.kvl = clampi(a.kv_len[it.s], 0, a.max_pages * a.page_size);
    const int i0 = r * a.tile_q;
    const int* list = a.plan + L.list + (int64_t)u * a.nkt;

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

    u32x4 kr[KPT], vr[KPT];
    auto load_tile = [&](int vt) {
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const int kappa = st_kg * KPT + k;
        const uint16_t* kp = key_row<HD>(a, kcache, knew, vt, kappa, it);
        const uint16_t* vp = key_row<HD>(a, vcache, vnew, vt, kappa, it);
        kr[k] = kp ? *(const u32x4*)(kp + 8 * st_c) : u32x4{0, 0, 0, 0};
        vr[k] = vp ? *(const u32x4*)(vp + 8 * st_c) : u32x4{0, 0, 0, 0};
      }
    };
    auto store_tile = [&](int buf, int vt, bool partial) {
#pragma unroll
      for (int k = 0; k < KPT; ++k) *(u32x4*)&sm.k[buf][st_kg * KPT + k][8 * st_c] = kr[k];
      const int pos0 = vt_pos(st_kg * KPT);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * st_c + e;
        unsigned h[KPT];
#pragma unroll
        for (int k = 0; k < KPT; ++k) h[k] = (e & 1) ? (vr[k][e >> 1] >> 16) : (vr[k][e >> 1] & 0xFFFFu);
        if constexpr (KPT == 4) {
          u32x2 pk = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          *(u32x2*)&sm.vt[buf][vt_off(d, pos0)] = pk;
        } else {
          *(unsigned*)&sm.vt[buf][vt_off(d, pos0)] = h[0] | (h[1] << 16);
        }
      }
      if (partial && tid < kTileK) sm.kblk[buf][tid] = key_block(a, vt, tid, it);
    };

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
    if (ob < oe) {
      const int e0 = list[ob];
      load_tile(e0 >> 1);
      store_tile(0, e0 >> 1, e0 & 1);
    }
    __syncthreads();

    for (int oi = ob; oi < oe; ++oi) {
      const int buf = (oi - ob) & 1;
      const bool partial = list[oi] & 1;
      const bool has_next = oi + 1 < oe;
      const int e_next = has_next ? list[oi + 1] : 0;
      if (has_next) load_tile(e_next >> 1);   // global loads in flight during the math below
      n_partial += partial;

      // S^T = K Q^T for two 32-key blocks x two 32-query blocks.
      f32x16 sc[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[qb][kb] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 kf = *(const bf16x8*)&sm.k[buf][32 * kb + col][16 * t + 8 * hl];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const bf16x8 qf = *(const bf16x8*)&sm.q[wave * 64 + qb * 32 + col][16 * t + 8 * hl];
            sc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, sc[qb][kb], 0, 0, 0);
          }
        }
      }

      // Mask, only on partial tiles. Lane (col, hl) holds key 32kb + 8(v/4) + 4hl + v%4.
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            const i32x4 kbv = *(const i32x4*)&sm.kblk[buf][32 * kb + 8 * v4 + 4 * hl];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (kbv[c] > qblk[qb]) sc[qb][kb][4 * v4 + c] = -INFINITY;
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
        const float mnew = fmaxf(m[qb], mx * sl2);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - muse);
        m[qb] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[qb][kb][v], sl2, -muse));
            sc[qb][kb][v] = p;
            rs += p;
          }
        l[qb] = l[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
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

      // O^T += V^T P^T: the 8 keys of step (kb, hs) for lane half hl sit contiguously at
      // transposed position 16*(2kb+hs) + 8*hl.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            const bf16x8 vf = *(const bf16x8*)&sm.vt[buf][vt_off(32 * db + col, 16 * (2 * kb + hs) + 8 * hl)];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][hs], o[qb][db], 0, 0, 0);
          }

      if (has_next) store_tile(buf ^ 1, e_next >> 1, e_next & 1);
      __syncthreads();
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
