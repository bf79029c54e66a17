// C ABI of the block-causal paged attention library: argument validation, the checked
// mode ("Paged Attention" asks for strict error checking of the page table), workspace
// layout and kernel dispatch. The declarations and their contracts are in include/bcp.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>
#include <vector>

#include "bcp_internal.h"

using namespace bcp;

// Scratch of the allocation-free attention entry point: the split-KV partial results and,
// when the caller passes no plan, the plan. The runtime places one copy of the array in the
// memory of every GPU that runs the library's code, for the life of the process. In host
// code `scratch` names a host-side stand-in, not device memory: host code reaches a GPU's
// copy only through the address hipGetSymbolAddress returns with that GPU current.
static __device__ __align__(256) unsigned char scratch[BCP_NOALLOC_SCRATCH_BYTES];

// A captured step: the HIP graph and its executable instance.
struct bcp_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BCP_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Geo {
  int G, tq, tk, nqt, nct, nlt, nkt;
  bool mode_b;
};

int check_meta(const bcp_meta* m, Geo* g) {
  if (!m) return fail(BCP_E_ARG, "meta is NULL");
  if (m->struct_size != sizeof(bcp_meta))
    return fail(BCP_E_ARG, "meta.struct_size is %u, expected %zu", m->struct_size, sizeof(bcp_meta));
  if (m->dtype != BCP_BF16 && m->dtype != BCP_F32) return fail(BCP_E_ARG, "dtype %d unknown", m->dtype);
  if (m->batch < 1) return fail(BCP_E_ARG, "batch must be >= 1 (got %d)", m->batch);
  if (m->num_q_heads < 1 || m->num_kv_heads < 1)
    return fail(BCP_E_ARG, "head counts must be >= 1 (Hq %d, Hkv %d)", m->num_q_heads, m->num_kv_heads);
  if (m->num_q_heads % m->num_kv_heads)
    return fail(BCP_E_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", m->num_q_heads,
                m->num_kv_heads);
  if (!m->cu_q || !m->kv_len || !m->page_table)
    return fail(BCP_E_ARG, "cu_q, kv_len and page_table must be non-NULL");
  if (!aligned(m->cu_q, 4) || !aligned(m->kv_len, 4) || !aligned(m->page_table, 4))
    return fail(BCP_E_ARG, "metadata arrays must be 4-byte aligned");
  if ((m->q_blk == nullptr) != (m->kv_blk == nullptr))
    return fail(BCP_E_ARG, "q_blk and kv_blk must be both set (mode B) or both NULL (mode A)");
  if (!m->q_blk && m->block_size < 1) return fail(BCP_E_ARG, "block_size must be >= 1 (got %d)", m->block_size);
  if (m->page_size < 1 || m->num_pages < 1 || m->max_pages_per_seq < 1)
    return fail(BCP_E_ARG, "page_size, num_pages and max_pages_per_seq must be >= 1");
  if (m->max_q_len < 0 || m->total_q < 0 || m->max_kv_len < 0)
    return fail(BCP_E_ARG, "max_q_len, total_q and max_kv_len must be >= 0");
  if ((int64_t)m->total_q > (int64_t)m->batch * m->max_q_len)
    return fail(BCP_E_ARG, "total_q %d exceeds batch * max_q_len", m->total_q);
  if ((int64_t)m->max_kv_len > (int64_t)m->max_pages_per_seq * m->page_size)
    return fail(BCP_E_ARG, "max_kv_len %d exceeds max_pages_per_seq * page_size", m->max_kv_len);
  if (m->flags & ~(BCP_F_CHECK | BCP_F_LIVE_IN_CACHE)) return fail(BCP_E_ARG, "unknown flags 0x%x", m->flags);
  if ((int64_t)m->num_pages * m->page_size > INT32_MAX || (int64_t)m->batch * m->max_pages_per_seq > INT32_MAX ||
      (int64_t)m->max_pages_per_seq * m->page_size > INT32_MAX)
    return fail(BCP_E_ARG, "pool, page table or per-sequence capacity too large for 32-bit row indices");
  if (m->window < 0) return fail(BCP_E_ARG, "window must be >= 0 (got %d)", m->window);
  if (m->window > 0 && m->q_blk && (!m->q_pos || !m->kv_pos))
    return fail(BCP_E_ARG, "a sliding window in mode B needs q_pos and kv_pos");
  if (m->window > 0 && m->q_blk && (!aligned(m->q_pos, 4) || !aligned(m->kv_pos, 4)))
    return fail(BCP_E_ARG, "q_pos and kv_pos must be 4-byte aligned");
  g->G = m->num_q_heads / m->num_kv_heads;
  g->mode_b = m->q_blk != nullptr;
  // Short live blocks (at most kNarrowRows packed rows per sequence and kv head, bf16) get
  // narrow q-tiles by default, which the narrow attention kernel handles.
  const bool narrow = m->dtype == BCP_BF16 && kNarrowRows % g->G == 0 &&
                      (int64_t)m->max_q_len * g->G <= kNarrowRows;
  g->tq = m->tile_q ? m->tile_q : std::max(1, (narrow ? kNarrowRows : kRowsPerWG) / g->G);
  g->tk = m->tile_k ? m->tile_k : kTileK;
  if (g->tq < 1 || g->tq > 4096 || g->tk < 1 || g->tk > 4096)
    return fail(BCP_E_ARG, "tile sizes must lie in [1, 4096] (tile_q %d, tile_k %d)", g->tq, g->tk);
  g->nqt = (int)ceil_div(m->max_q_len, g->tq);
  g->nct = (int)ceil_div(m->max_kv_len, g->tk);
  g->nlt = (int)ceil_div(m->max_q_len, g->tk);
  g->nkt = g->nct + g->nlt;
  if ((int64_t)m->batch * g->nqt * g->nkt * 2 + 64 > INT32_MAX)
    return fail(BCP_E_ARG, "tile grid too large");
  if (g->mode_b && m->window > 0 && g->nkt > kMaxBandKeyTiles)
    return fail(BCP_E_UNSUPPORTED, "a window in mode B supports at most %d key tiles (got %d)", kMaxBandKeyTiles,
                g->nkt);
  return BCP_OK;
}

int check_attention_shape(const bcp_meta* m, const Geo& g) {
  if (m->head_dim != 64 && m->head_dim != 128)
    return fail(BCP_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", m->head_dim);
  if (kRowsPerWG % g.G)
    return fail(BCP_E_UNSUPPORTED, "query heads per kv head (%d) must divide %d", g.G, kRowsPerWG);
  const bool narrow_ok = m->dtype == BCP_BF16 && kNarrowRows % g.G == 0 && g.tq == kNarrowRows / g.G;
  if ((g.tq != kRowsPerWG / g.G && !narrow_ok) || g.tk != kTileK)
    return fail(BCP_E_UNSUPPORTED, "attention needs tile_q = %d (or %d for bf16) and tile_k = %d (got %d, %d)",
                kRowsPerWG / g.G, kNarrowRows / g.G, kTileK, g.tq, g.tk);
  return BCP_OK;
}

template <class T>
int copy_to_host(std::vector<T>& v, const T* src, size_t n, hipStream_t stream) {
  v.resize(n);
  if (!n) return BCP_OK;
  hipError_t e = hipMemcpyAsync(v.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "checked mode: hipMemcpyAsync");
  return BCP_OK;
}

// Checked mode copies to the host, which a stream under capture cannot do.
int refuse_if_capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (st != hipStreamCaptureStatusNone) return fail(BCP_E_ARG, "checked mode cannot run on a stream under capture");
  return BCP_OK;
}

// Checked mode: the metadata the kernels will read, validated on the host. *len_hash (when
// given) receives the hash of the sequences' live rows and committed lengths that the
// planner records in a plan's header.
int validate_metadata(const bcp_meta* m, hipStream_t stream, uint32_t* len_hash = nullptr) {
  if (int rc = refuse_if_capturing(stream)) return rc;
  std::vector<int32_t> cu, kvl, pt, qb, kb;
  int rc;
  if ((rc = copy_to_host(cu, m->cu_q, m->batch + 1, stream))) return rc;
  if ((rc = copy_to_host(kvl, m->kv_len, m->batch, stream))) return rc;
  if ((rc = copy_to_host(pt, m->page_table, (size_t)m->batch * m->max_pages_per_seq, stream))) return rc;
  if (m->q_blk) {
    if ((rc = copy_to_host(qb, m->q_blk, m->total_q, stream))) return rc;
    if ((rc = copy_to_host(kb, m->kv_blk, (size_t)m->num_pages * m->page_size, stream))) return rc;
  }
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "checked mode: hipStreamSynchronize");
  if (cu[0] != 0) return fail(BCP_E_RANGE, "cu_q[0] = %d, expected 0", cu[0]);
  for (int s = 0; s < m->batch; ++s) {
    const int ql = cu[s + 1] - cu[s];
    if (ql < 0 || ql > m->max_q_len)
      return fail(BCP_E_RANGE, "sequence %d: q_len %d outside [0, max_q_len %d]", s, ql, m->max_q_len);
    if (kvl[s] < 0 || kvl[s] > m->max_kv_len)
      return fail(BCP_E_RANGE, "sequence %d: kv_len %d outside [0, max_kv_len %d]", s, kvl[s], m->max_kv_len);
    // Pages of the committed rows, and of the live rows when those are read from the pool.
    const int64_t rows = kvl[s] + ((m->flags & BCP_F_LIVE_IN_CACHE) ? ql : 0);
    if (rows > (int64_t)m->max_pages_per_seq * m->page_size)
      return fail(BCP_E_RANGE, "sequence %d: kv_len + q_len = %lld exceeds the page table", s, (long long)rows);
    for (int64_t lp = 0; lp < ceil_div(rows, m->page_size); ++lp) {
      const int p = pt[(size_t)s * m->max_pages_per_seq + lp];
      if (p < 0 || p >= m->num_pages)
        return fail(BCP_E_RANGE, "sequence %d: page_table[%lld] = %d outside [0, %d)", s, (long long)lp, p,
                    m->num_pages);
      if (m->q_blk) {
        for (int k = 0; k < m->page_size && lp * m->page_size + k < kvl[s]; ++k) {
          const int b = kb[(size_t)p * m->page_size + k];
          if (b == kNegInfBlk || b == kNoKeyBlk)
            return fail(BCP_E_RANGE, "sequence %d: kv_blk of row %lld is a reserved value", s,
                        (long long)(lp * m->page_size + k));
        }
      }
    }
  }
  if (cu[m->batch] != m->total_q)
    return fail(BCP_E_RANGE, "cu_q[batch] = %d but total_q = %d", cu[m->batch], m->total_q);
  for (int i = 0; i < (int)qb.size(); ++i)
    if (qb[i] == kNegInfBlk || qb[i] >= kNoKeyBlk - 1)
      return fail(BCP_E_RANGE, "q_blk[%d] is a reserved value", i);
  if (len_hash) {
    const int64_t cap = (int64_t)m->max_pages_per_seq * m->page_size;
    uint32_t h = 0;
    for (int s = 0; s < m->batch; ++s)
      h += seq_len_hash(s, cu[s], cu[s + 1] - cu[s], (int)std::min<int64_t>(kvl[s], cap));
    *len_hash = h;
  }
  return BCP_OK;
}

// Checked mode: a caller's plan must have been built by build_tile_mask for this step --
// the same shapes, window and mode, and the same live rows and committed lengths.
int validate_plan(const bcp_meta* m, const Geo& g, const void* plan, uint32_t len_hash, hipStream_t stream) {
  int32_t h[kHdrWords];
  hipError_t e = hipMemcpyAsync(h, plan, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "checked mode: reading the plan header");
  if (h[kHdrMagic] != kPlanMagic) return fail(BCP_E_ARG, "plan was not written by build_tile_mask");
  if (h[kHdrTileQ] != g.tq || h[kHdrTileK] != g.tk || h[kHdrNqt] != g.nqt || h[kHdrNkt] != g.nkt ||
      h[kHdrBatch] != m->batch || h[kHdrHkv] != m->num_kv_heads || h[kHdrWindow] != m->window ||
      h[kHdrModeB] != (g.mode_b ? 1 : 0) || h[kHdrTotalQ] != m->total_q ||
      h[kHdrKvCap] != m->max_pages_per_seq * m->page_size)
    return fail(BCP_E_ARG,
                "plan was built for another step shape (plan: batch %d, Hkv %d, tiles %dx%d, grid %dx%d, "
                "window %d, mode %s, total_q %d, capacity %d; meta: batch %d, Hkv %d, tiles %dx%d, grid %dx%d, "
                "window %d, mode %s, total_q %d, capacity %d)",
                h[kHdrBatch], h[kHdrHkv], h[kHdrTileQ], h[kHdrTileK], h[kHdrNqt], h[kHdrNkt], h[kHdrWindow],
                h[kHdrModeB] ? "B" : "A", h[kHdrTotalQ], h[kHdrKvCap], m->batch, m->num_kv_heads, g.tq, g.tk,
                g.nqt, g.nkt, m->window, g.mode_b ? "B" : "A", m->total_q, m->max_pages_per_seq * m->page_size);
  if ((uint32_t)h[kHdrLenHash] != len_hash)
    return fail(BCP_E_ARG, "plan was built for other live rows or committed lengths (a stale plan?)");
  return BCP_OK;
}

// Compute units of the current device, cached per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Device address of the current GPU's copy of `scratch`, looked up once per device.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(BCP_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p) return fail(BCP_E_HIP, "hipGetSymbolAddress(scratch) gave NULL");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BCP_OK;
}

size_t plan_bytes_for(const bcp_meta* m, const Geo& g) {
  return (size_t)plan_layout(m->batch, g.nqt, g.nkt, m->num_kv_heads).words * sizeof(int32_t);
}

// Partial results are needed only if a (unit, kv head) pair can be cut by a range
// boundary, i.e. if it can have more than one tile.
size_t partial_bytes_for(const bcp_meta* m, const Geo& g) {
  if (g.nkt <= 1) return 0;
  return (size_t)kMaxPartialSlots * kRowsPerWG * (m->head_dim + 1) * sizeof(float);
}

ClassifyArgs classify_args(const bcp_meta* m, const Geo& g) {
  ClassifyArgs a{};
  a.cu_q = m->cu_q;
  a.kv_len = m->kv_len;
  a.page_table = m->page_table;
  a.q_blk = m->q_blk;
  a.kv_blk = m->kv_blk;
  a.batch = m->batch;
  a.total_q = m->total_q;
  a.tile_q = g.tq;
  a.tile_k = g.tk;
  a.nqt = g.nqt;
  a.nct = g.nct;
  a.nkt = g.nkt;
  a.block_size = g.mode_b ? 1 : m->block_size;
  a.page_size = m->page_size;
  a.num_pages = m->num_pages;
  a.max_pages = m->max_pages_per_seq;
  a.max_q_len = m->max_q_len;
  a.mode_b = g.mode_b;
  a.phys_per_tile = std::max(1, g.tk / m->page_size);
  a.phys_tiles = g.nct;
  a.num_kv_heads = m->num_kv_heads;
  a.window = m->window;
  if (g.mode_b && m->window > 0) {
    a.q_pos = m->q_pos;
    a.kv_pos = m->kv_pos;
  }
  return a;
}

int run_classify_and_plan(const bcp_meta* m, const Geo& g, uint8_t* tile_class, int32_t* phys_page,
                          int32_t* plan, hipStream_t stream) {
  ClassifyArgs a = classify_args(m, g);
  a.tile_class = tile_class;
  a.phys_page = phys_page;
  a.plan = plan;
  a.grid_q = std::max(g.nqt, 1);
  PlanArgs p{};
  p.plan = plan;
  p.batch = m->batch;
  p.nqt = g.nqt;
  p.nkt = g.nkt;
  p.num_kv_heads = m->num_kv_heads;
  p.tile_q = g.tq;
  p.tile_k = g.tk;
  p.cu_q = m->cu_q;
  p.kv_len = m->kv_len;
  p.total_q = m->total_q;
  p.max_q_len = m->max_q_len;
  p.kv_cap = m->max_pages_per_seq * m->page_size;
  p.window = m->window;
  p.mode_b = g.mode_b ? 1 : 0;
  // A small mode-A step (with or without a window) is classified by the planner itself: one
  // launch.
  const int64_t elems = (int64_t)m->batch * g.nqt * g.nkt + (phys_page ? (int64_t)m->batch * g.nct * a.phys_per_tile : 0);
  if (plan && !g.mode_b && m->batch <= 1024 && elems <= kFusedPlanElems) {
    p.fused = 1;
    p.nct = g.nct;
    p.block_size = m->block_size;
    p.page_size = m->page_size;
    p.num_pages = m->num_pages;
    p.max_pages = m->max_pages_per_seq;
    p.phys_per_tile = a.phys_per_tile;
    p.tile_class = tile_class;
    p.phys_page = phys_page;
    p.page_table = m->page_table;
    hipError_t e = launch_planner(p, stream);
    if (e != hipSuccess) return hip_fail(e, "launch planner");
    return BCP_OK;
  }
  hipError_t e = launch_classify(a, stream);
  if (e != hipSuccess) return hip_fail(e, "launch classify");
  if (plan) {
    e = launch_planner(p, stream);
    if (e != hipSuccess) return hip_fail(e, "launch planner");
  }
  return BCP_OK;
}

}  // namespace

extern "C" {

int bcp_abi_version(void) { return BCP_ABI_VERSION; }

const char* bcp_last_error(void) { return g_err.c_str(); }

int bcp_graph_begin(hipStream_t stream) {
  hipError_t e = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  g_err.clear();
  return BCP_OK;
}

int bcp_graph_end(hipStream_t stream, bcp_graph** graph) {
  if (!graph) return fail(BCP_E_ARG, "bcp_graph_end: graph is NULL");
  *graph = nullptr;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(stream, &g);
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  bcp_graph* r = new (std::nothrow) bcp_graph{g, x};
  if (!r) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return fail(BCP_E_ARG, "bcp_graph_end: out of host memory");
  }
  *graph = r;
  g_err.clear();
  return BCP_OK;
}

int bcp_graph_launch(bcp_graph* graph, hipStream_t stream) {
  if (!graph) return fail(BCP_E_ARG, "bcp_graph_launch: graph is NULL");
  hipError_t e = hipGraphLaunch(graph->exec, stream);
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  g_err.clear();
  return BCP_OK;
}

void bcp_graph_destroy(bcp_graph* graph) {
  if (!graph) return;
  (void)hipGraphExecDestroy(graph->exec);
  (void)hipGraphDestroy(graph->graph);
  delete graph;
}

int32_t bcp_num_q_tiles(const bcp_meta* m) {
  Geo g;
  return check_meta(m, &g) == BCP_OK ? g.nqt : 0;
}

int32_t bcp_num_k_tiles(const bcp_meta* m) {
  Geo g;
  return check_meta(m, &g) == BCP_OK ? g.nkt : 0;
}

size_t bcp_plan_size(const bcp_meta* m) {
  Geo g;
  if (check_meta(m, &g) != BCP_OK) return 0;
  return plan_bytes_for(m, g);
}

int build_tile_mask(const bcp_meta* m, uint8_t* tile_class, int32_t* phys_page, void* plan,
                    size_t plan_bytes, hipStream_t stream) {
  Geo g;
  int rc = check_meta(m, &g);
  if (rc) return rc;
  if (!tile_class && !phys_page && !plan)
    return fail(BCP_E_ARG, "build_tile_mask: tile_class, phys_page and plan are all NULL");
  if (plan && plan_bytes < plan_bytes_for(m, g))
    return fail(BCP_E_WORKSPACE, "plan buffer has %zu bytes, needs %zu", plan_bytes, plan_bytes_for(m, g));
  if ((plan && !aligned(plan, 16)) || (phys_page && !aligned(phys_page, 4)))
    return fail(BCP_E_ARG, "plan must be 16-byte and phys_page 4-byte aligned");
  if (m->flags & BCP_F_CHECK) {
    if ((rc = validate_metadata(m, stream))) return rc;
  }
  g_err.clear();
  return run_classify_and_plan(m, g, tile_class, phys_page, (int32_t*)plan, stream);
}

size_t attn_block_causal_paged_workspace_size(const bcp_meta* m) {
  Geo g;
  if (check_meta(m, &g) != BCP_OK) return 0;
  if (m->head_dim != 64 && m->head_dim != 128) return 0;
  const size_t part = partial_bytes_for(m, g);
  return part + plan_bytes_for(m, g) + 256;
}

}  // extern "C"

namespace {

// The attention call. With noalloc the workspace is this GPU's copy of `scratch` (the
// workspace arguments are ignored), found after every host-side check has passed.
int attn_impl(const bcp_meta* m, const void* q, const void* k_new, const void* v_new, const void* k_cache,
              const void* v_cache, const void* plan, float scale, void* out, float* lse, void* workspace,
              size_t workspace_bytes, uint64_t* stats, hipStream_t stream, bool noalloc) {
  Geo g;
  int rc = check_meta(m, &g);
  if (rc) return rc;
  if ((rc = check_attention_shape(m, g))) return rc;
  const bool in_place = (m->flags & BCP_F_LIVE_IN_CACHE) != 0;
  if (in_place) k_new = v_new = nullptr;   // not read: the live rows come from the pool
  if (!q || (!in_place && (!k_new || !v_new)) || !k_cache || !v_cache || !out)
    return fail(BCP_E_ARG, "q, k_new, v_new, k_cache, v_cache and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4)) ||
      (plan && !aligned(plan, 16)) || (stats && !aligned(stats, 8)))
    return fail(BCP_E_ARG, "tensors must be 16-byte aligned (lse 4, stats 8)");
  if (!std::isfinite(scale)) return fail(BCP_E_ARG, "scale is not finite");
  const size_t part = partial_bytes_for(m, g);
  const size_t need = part + (plan ? 0 : plan_bytes_for(m, g) + 256);
  if (noalloc) {
    if (need > (size_t)BCP_NOALLOC_SCRATCH_BYTES)
      return fail(BCP_E_WORKSPACE,
                  "the allocation-free call needs %zu bytes of scratch (%s), more than its %zu; pass a plan "
                  "from build_tile_mask or use attn_block_causal_paged with a workspace",
                  need, plan ? "split-KV partials" : "split-KV partials and the plan", (size_t)BCP_NOALLOC_SCRATCH_BYTES);
  } else {
    if (workspace_bytes < need || (need && !workspace))
      return fail(BCP_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (workspace && !aligned(workspace, 16)) return fail(BCP_E_ARG, "workspace must be 16-byte aligned");
  }
  if (m->flags & BCP_F_CHECK) {
    uint32_t len_hash = 0;
    if ((rc = validate_metadata(m, stream, &len_hash))) return rc;
    if (plan && (rc = validate_plan(m, g, plan, len_hash, stream))) return rc;
  }
  if (noalloc && need) {
    if ((rc = scratch_address(&workspace))) return rc;
    workspace_bytes = BCP_NOALLOC_SCRATCH_BYTES;
  }
  g_err.clear();
  if (m->total_q == 0 || g.nqt == 0) return BCP_OK;

  char* ws = (char*)workspace;
  const int32_t* plan_ptr = (const int32_t*)plan;
  if (!plan_ptr) {
    int32_t* own = (int32_t*)(ws + part);
    own = (int32_t*)(((uintptr_t)own + 255) & ~(uintptr_t)255);
    if ((rc = run_classify_and_plan(m, g, nullptr, nullptr, own, stream))) return rc;
    plan_ptr = own;
  }

  AttnArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.lse = lse;
  // Split-KV partials: fp32 for fp32 steps; for bf16 steps fp16 rows in the first half of the
  // same region and their row factors right after them (the fp32-sized region holds both).
  const size_t part_elems = (size_t)kMaxPartialSlots * kRowsPerWG * m->head_dim;
  const bool half_parts = m->dtype == BCP_BF16;
  a.part_o = part && !half_parts ? (float*)ws : nullptr;
  a.part_h = part && half_parts ? (uint16_t*)ws : nullptr;
  a.part_scale = part && half_parts ? (float*)((uint16_t*)ws + part_elems) : nullptr;
  a.part_lse = part ? (float*)ws + part_elems : nullptr;
  a.cu_q = m->cu_q;
  a.kv_len = m->kv_len;
  a.page_table = m->page_table;
  a.q_blk = m->q_blk;
  a.kv_blk = m->kv_blk;
  a.plan = plan_ptr;
  a.stats = (unsigned long long*)stats;
  a.batch = m->batch;
  a.total_q = m->total_q;
  a.max_q_len = m->max_q_len;
  a.Hq = m->num_q_heads;
  a.Hkv = m->num_kv_heads;
  a.G = g.G;
  a.tile_q = g.tq;
  a.nqt = g.nqt;
  a.nkt = g.nkt;
  a.nct = g.nct;
  a.page_size = m->page_size;
  a.num_pages = m->num_pages;
  a.max_pages = m->max_pages_per_seq;
  a.block_size = g.mode_b ? 1 : m->block_size;
  a.mode_b = g.mode_b;
  a.max_items = plan_layout(m->batch, g.nqt, g.nkt, m->num_kv_heads).max_items;
  a.page_shift = (m->page_size & (m->page_size - 1)) ? -1 : __builtin_ctz((unsigned)m->page_size);
  a.window = m->window;
  if (g.mode_b && m->window > 0) {
    a.q_pos = m->q_pos;
    a.kv_pos = m->kv_pos;
  }
  a.live_in_cache = (m->flags & BCP_F_LIVE_IN_CACHE) != 0;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)m->head_dim);
  a.scale_log2 = sc * 1.4426950408889634f;

  const int cus = device_cus();
  const int grid = kWGs;   // one workgroup per range of the plan
  const bool narrow = m->dtype == BCP_BF16 && g.tq * g.G == kNarrowRows;
  hipError_t e = m->dtype != BCP_BF16 ? launch_attn_f32(a, m->head_dim, grid, stream)
                 : narrow             ? launch_attn_bf16_narrow(a, m->head_dim, grid, stream)
                                      : launch_attn_bf16(a, m->head_dim, grid, stream);
  if (e != hipSuccess) return hip_fail(e, "launch attention");
  if (part) {
    const int cgrid = (int)std::min<int64_t>((int64_t)kMaxPartialSlots * 16, (int64_t)cus * 8);
    e = launch_combine(a, m->head_dim, m->dtype == BCP_BF16, cgrid, stream);
    if (e != hipSuccess) return hip_fail(e, "launch combine");
  }
  return BCP_OK;
}

}  // namespace

extern "C" {

int attn_block_causal_paged(const bcp_meta* m, const void* q, const void* k_new, const void* v_new,
                            const void* k_cache, const void* v_cache, const void* plan, float scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            uint64_t* stats, hipStream_t stream) {
  return attn_impl(m, q, k_new, v_new, k_cache, v_cache, plan, scale, out, lse, workspace, workspace_bytes,
                   stats, stream, false);
}

int attn_block_causal_paged_noalloc(const bcp_meta* m, const void* q, const void* k_new, const void* v_new,
                                    const void* k_cache, const void* v_cache, const void* plan, float scale,
                                    void* out, float* lse, uint64_t* stats, hipStream_t stream) {
  return attn_impl(m, q, k_new, v_new, k_cache, v_cache, plan, scale, out, lse, nullptr, 0, stats, stream, true);
}

int kv_commit_block(const bcp_meta* m, const void* k_src, const void* v_src, const int32_t* cu_src,
                    const int32_t* src_row, const int32_t* dst_start, const int32_t* src_blk,
                    int32_t total_commit, int32_t n_src, void* k_cache, void* v_cache,
                    int32_t* kv_blk_out, hipStream_t stream) {
  if (!m) return fail(BCP_E_ARG, "meta is NULL");
  if (m->struct_size != sizeof(bcp_meta)) return fail(BCP_E_ARG, "meta.struct_size mismatch");
  if (m->dtype != BCP_BF16 && m->dtype != BCP_F32) return fail(BCP_E_ARG, "dtype %d unknown", m->dtype);
  if (m->batch < 1 || m->num_kv_heads < 1 || m->head_dim < 1)
    return fail(BCP_E_ARG, "batch, num_kv_heads and head_dim must be >= 1");
  if (m->page_size < 1 || m->num_pages < 1 || m->max_pages_per_seq < 1 || !m->page_table)
    return fail(BCP_E_ARG, "page geometry invalid or page_table NULL");
  if (total_commit < 0 || n_src < 0) return fail(BCP_E_ARG, "total_commit and n_src must be >= 0");
  const int esize = m->dtype == BCP_BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)m->num_kv_heads * m->head_dim * esize;
  if (row_bytes % 16) return fail(BCP_E_UNSUPPORTED, "a cache row (%lld bytes) must be a multiple of 16 bytes",
                                  (long long)row_bytes);
  if ((k_src == nullptr) != (v_src == nullptr)) return fail(BCP_E_ARG, "k_src and v_src must be both set or both NULL");
  if (!k_cache || !v_cache || !cu_src || !dst_start)
    return fail(BCP_E_ARG, "cu_src, dst_start, k_cache and v_cache must be non-NULL");
  if (!k_src && (src_blk == nullptr) != (kv_blk_out == nullptr))
    return fail(BCP_E_ARG, "a commit without k_src/v_src moves tags only: src_blk and kv_blk_out go together");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || (k_src && !aligned(k_src, 16)) ||
      (v_src && !aligned(v_src, 16)))
    return fail(BCP_E_ARG, "K/V buffers must be 16-byte aligned");
  if (m->flags & BCP_F_CHECK) {
    std::vector<int32_t> cu, rows, dst, pt;
    int rc;
    if ((rc = refuse_if_capturing(stream))) return rc;
    if ((rc = copy_to_host(cu, cu_src, m->batch + 1, stream))) return rc;
    if ((rc = copy_to_host(dst, dst_start, m->batch, stream))) return rc;
    if ((rc = copy_to_host(pt, m->page_table, (size_t)m->batch * m->max_pages_per_seq, stream))) return rc;
    if (src_row && (rc = copy_to_host(rows, src_row, total_commit, stream))) return rc;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "checked mode: hipStreamSynchronize");
    if (cu[0] != 0 || cu[m->batch] != total_commit)
      return fail(BCP_E_RANGE, "cu_src must start at 0 and end at total_commit %d", total_commit);
    std::unordered_set<int64_t> seen;
    for (int s = 0; s < m->batch; ++s) {
      if (cu[s + 1] < cu[s]) return fail(BCP_E_RANGE, "cu_src decreases at sequence %d", s);
      for (int r = 0; r < cu[s + 1] - cu[s]; ++r) {
        const int src = src_row ? rows[cu[s] + r] : cu[s] + r;
        if (src < 0 || src >= n_src) return fail(BCP_E_RANGE, "sequence %d: source row %d outside [0, %d)", s, src, n_src);
        const int64_t j = (int64_t)dst[s] + r;
        if (j < 0 || j >= (int64_t)m->max_pages_per_seq * m->page_size)
          return fail(BCP_E_RANGE, "sequence %d: destination row %lld outside the page table", s, (long long)j);
        const int p = pt[(size_t)s * m->max_pages_per_seq + j / m->page_size];
        if (p < 0 || p >= m->num_pages)
          return fail(BCP_E_RANGE, "sequence %d: destination page %d outside [0, %d)", s, p, m->num_pages);
        const int64_t slot = (int64_t)p * m->page_size + j % m->page_size;
        if (!seen.insert(slot).second)
          return fail(BCP_E_RANGE, "two rows commit to page %d slot %lld", p, (long long)(j % m->page_size));
      }
    }
  }
  g_err.clear();
  if (total_commit == 0 || (!k_src && !kv_blk_out)) return BCP_OK;   // nothing to move
  CommitArgs a{};
  a.k_src = k_src;
  a.v_src = v_src;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cu_src = cu_src;
  a.src_row = src_row;
  a.dst_start = dst_start;
  a.src_blk = src_blk;
  a.kv_blk_out = kv_blk_out;
  a.page_table = m->page_table;
  a.batch = m->batch;
  a.total = total_commit;
  a.n_src = n_src;
  a.row_chunks = (int)(row_bytes / 16);
  a.page_size = m->page_size;
  a.num_pages = m->num_pages;
  a.max_pages = m->max_pages_per_seq;
  const int grid = std::max(1, std::min(total_commit, device_cus() * 16));
  hipError_t e = launch_commit(a, grid, stream);
  if (e != hipSuccess) return hip_fail(e, "launch commit");
  return BCP_OK;
}

}  // extern "C"
