// KV commit: finished rows copied bit for bit into their cache pages.
//
// "Inference for Interpretable Text-Diffusion Models", section "KV Cache", step 3: the keys
// and values of a block go to the cache in a pass of their own once all of its positions are
// decided; section "Paged Attention": logical row j of sequence s lives in page
// page_table[s, j/P], slot j%P.
// "Inference: Fewer, smaller forwards", Advancement 11: arena entries carry their position
// tag, recorded here as the block id next to the slot.
//
// The copy is pure data movement: each thread moves 16-byte vectors of one row (the
// Hkv*d contiguous elements of one source row map onto one contiguous destination slot),
// so reads and writes are fully coalesced. A workgroup walks rows in a grid-stride loop;
// the row's sequence comes from a binary search of cu_src (uniform per workgroup), which
// with the destination starts is staged in LDS first when the batch fits, so a row waits
// for three dependent loads (those arrays, its page, its data) rather than one per step
// of the search.
#include "bcp_internal.h"

namespace bcp {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kCommitLdsSeqs = 2048;

__global__ __launch_bounds__(256) void commit_kernel(CommitArgs a) {
  const u32x4* ks = (const u32x4*)a.k_src;
  const u32x4* vs = (const u32x4*)a.v_src;
  u32x4* kc = (u32x4*)a.k_cache;
  u32x4* vc = (u32x4*)a.v_cache;
  const int tid = threadIdx.x;
  __shared__ int s_cu[kCommitLdsSeqs + 1], s_dst[kCommitLdsSeqs];
  const bool in_lds = a.batch <= kCommitLdsSeqs;
  if (in_lds) {
    for (int i = tid; i <= a.batch; i += blockDim.x) s_cu[i] = a.cu_src[i];
    for (int i = tid; i < a.batch; i += blockDim.x) s_dst[i] = a.dst_start[i];
    __syncthreads();
  }
  auto cu = [&](int i) { return in_lds ? s_cu[i] : a.cu_src[i]; };
  for (int row = blockIdx.x; row < a.total; row += gridDim.x) {
    const int src = a.src_row ? a.src_row[row] : row;
    // Sequence of this commit row: the last s with cu_src[s] <= row.
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu(mid) <= row) lo = mid; else hi = mid;
    }
    const int s = lo;
    const int r = row - cu(s);
    const int j = (in_lds ? s_dst[s] : a.dst_start[s]) + r;
    const int page = translate_page(a.page_table, s, j, a.page_size, a.max_pages, a.num_pages);
    if (src < 0 || src >= a.n_src || page < 0 || r < 0) continue;   // out of range: no write
    const int64_t dst = (int64_t)page * a.page_size + (j % a.page_size);
    // Non-temporal loads and stores: every byte is moved once (measured: the C3 commit of
    // 32,768 rows 80 -> 60 us).
    for (int c = tid; c < 2 * a.row_chunks; c += blockDim.x) {
      if (c < a.row_chunks)
        __builtin_nontemporal_store(__builtin_nontemporal_load(ks + (int64_t)src * a.row_chunks + c), kc + dst * a.row_chunks + c);
      else
        __builtin_nontemporal_store(__builtin_nontemporal_load(vs + (int64_t)src * a.row_chunks + (c - a.row_chunks)), vc + dst * a.row_chunks + (c - a.row_chunks));
    }
    if (tid == 0 && a.kv_blk_out && a.src_blk) a.kv_blk_out[dst] = a.src_blk[src];
  }
}

// Commit of rows whose keys and values were already written into their slots: only the
// block ids move, one row per thread.
__global__ __launch_bounds__(256) void commit_ids_kernel(CommitArgs a) {
  for (int row = blockIdx.x * blockDim.x + threadIdx.x; row < a.total; row += gridDim.x * blockDim.x) {
    const int src = a.src_row ? a.src_row[row] : row;
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_src[mid] <= row) lo = mid; else hi = mid;
    }
    const int r = row - a.cu_src[lo];
    const int j = a.dst_start[lo] + r;
    const int page = translate_page(a.page_table, lo, j, a.page_size, a.max_pages, a.num_pages);
    if (src < 0 || src >= a.n_src || page < 0 || r < 0) continue;
    a.kv_blk_out[(int64_t)page * a.page_size + (j % a.page_size)] = a.src_blk[src];
  }
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, int grid, hipStream_t stream) {
  if (a.k_src)
    hipLaunchKernelGGL(commit_kernel, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(commit_ids_kernel, dim3((a.total + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bcp
