/*
 * bcp.h -- block-causal paged attention and KV commit for MI355X (gfx950).
 *
 * The operation (from "Inference for Interpretable Text-Diffusion Models", Background
 * and sections "FlexAttention with Aligned Tiles", "KV Cache", "Paged Attention"; and
 * "Inference: Fewer, smaller forwards", Advancements 1, 11 and 13):
 *
 *   A batch of sequences each has kv_len committed rows whose keys/values sit in a
 *   paged cache (fixed-size pages anywhere in a pool, located through a page table),
 *   and q_len live rows of the active block(s), whose queries, keys and values are
 *   passed in. Every live row attends
 *     mode A: to all committed rows, and to live row j iff j/D <= i/D (blocks of D rows
 *             counted from the sequence's first live row: bidirectional inside a block,
 *             causal across blocks, never to later blocks);
 *     mode B: to committed row j iff kv_blk[slot(j)] <= q_blk[i], and to live row j iff
 *             q_blk[j] <= q_blk[i] (block ids per row, as in multi-canvas decoding where
 *             canvas c sees the prompt, earlier canvases and itself);
 *   with a sliding window W, additionally only to keys at most W-1 positions before the
 *   query (mode A: committed row j at position j, live row i at kv_len + i; mode B: the
 *   positions q_pos and kv_pos give, as arena entries carry their absolute position).
 *   out = softmax(scale * q k^T restricted to visible keys) v, per query head, with
 *   grouped-query attention: query head h reads kv head h / (Hq / Hkv).
 *   When a block is finished its rows are committed: copied bit for bit into the page
 *   slots that follow the sequence's committed rows.
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer unless marked (host). All buffers are owned by
 *     the caller; the library allocates no device memory, keeps no pointer past a call
 *     and has no global state other than a thread-local error message and a per-device
 *     cache of the compute-unit count (the step-graph entry points below are the one
 *     exception: a graph holds the HIP graph it captured until it is destroyed).
 *   - Work is enqueued asynchronously on `stream`; no entry point synchronizes, except
 *     in checked mode (BCP_F_CHECK), which copies the metadata to the host once and
 *     validates it before launching anything.
 *   - Host-visible arguments are always validated before any launch. On a non-OK
 *     return nothing has been enqueued and no output was touched; bcp_last_error()
 *     describes the failure.
 *   - Device-side content (lengths, page ids, block ids, row indices) is validated only
 *     in checked mode. Without it, bad content gives unspecified results, but every
 *     kernel bounds-checks page ids and row indices, so it never reads or writes
 *     outside the buffers described here.
 *   - Tensors are dense, row-major, 16-byte aligned.
 */
#ifndef BCP_H
#define BCP_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BCP_ABI_VERSION 3

enum { BCP_BF16 = 0, BCP_F32 = 1 };
enum { BCP_TILE_SKIP = 0, BCP_TILE_PARTIAL = 1, BCP_TILE_FULL = 2 };
enum {
  BCP_OK = 0,
  BCP_E_ARG = 1,          /* malformed host argument (null, size, alignment, tile size) */
  BCP_E_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, dtype, group size) */
  BCP_E_RANGE = 3,        /* checked mode: device metadata out of range or duplicated */
  BCP_E_WORKSPACE = 4,    /* workspace or plan buffer too small */
  BCP_E_HIP = 5           /* a HIP runtime call failed */
};
#define BCP_F_CHECK 1u    /* validate device metadata before launch (one device->host sync) */
/* The live rows' keys and values already sit in the cache pool: live row i of sequence s
 * at logical row kv_len[s] + i, written there by whatever produced them ("Inference: Fewer,
 * smaller forwards", Advancement 11: the active block's entries live in the same arena as
 * the committed ones, so committing them is a length change). Attention then reads one
 * paged source of kv_len + q_len rows and ignores k_new/v_new (they may be NULL); the
 * commit of such rows moves only their block ids (k_src = v_src = NULL). Each sequence
 * needs pages mapped for its kv_len + q_len rows (checked mode verifies it). */
#define BCP_F_LIVE_IN_CACHE 2u

/*
 * Geometry of one step, shared by every call of the step (and every layer).
 * Layouts:
 *   q       [total_q, Hq, d]            live queries of the active blocks
 *   k_new   [total_q, Hkv, d]           live keys (positional encoding already applied)
 *   v_new   [total_q, Hkv, d]
 *   cache   [num_pages, page_size, Hkv, d]  one pool each for K and V (one layer)
 * Logical committed row j of sequence s lives in page page_table[s*max_pages_per_seq +
 * j/page_size], slot j%page_size ("Paged Attention": the page table maps the logical
 * layout onto physical pages).
 */
typedef struct bcp_meta {
  uint32_t struct_size;        /* sizeof(bcp_meta) */
  int32_t dtype;               /* BCP_BF16 or BCP_F32, for q, k/v (live and cache) and out */
  int32_t batch;               /* number of sequences, >= 1 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0 and 256 % (Hq/Hkv) == 0 */
  int32_t head_dim;            /* d: 64 or 128 */
  int32_t block_size;          /* D >= 1: live rows per block (mode A) */
  const int32_t* cu_q;         /* [batch+1] live-row offsets; cu_q[0] = 0, cu_q[batch] = total_q */
  const int32_t* q_blk;        /* [total_q] block id per live row, or NULL (mode A) */
  int32_t total_q;             /* host copy of cu_q[batch] */
  int32_t max_q_len;           /* host bound on cu_q[s+1]-cu_q[s] */
  const int32_t* kv_len;       /* [batch] committed rows per sequence */
  const int32_t* page_table;   /* [batch, max_pages_per_seq] physical page ids */
  const int32_t* kv_blk;       /* [num_pages*page_size] block id per cache slot, or NULL (mode A) */
  int32_t num_pages;           /* pool size in pages */
  int32_t page_size;           /* P >= 1 */
  int32_t max_pages_per_seq;   /* row stride of page_table */
  int32_t max_kv_len;          /* host bound on kv_len[s] */
  int32_t tile_q;              /* query positions per q-tile; 0 -> 256/(Hq/Hkv), or 64/(Hq/Hkv)
                                  for bf16 steps with max_q_len*(Hq/Hkv) <= 64 (short live
                                  blocks such as a causal extend: "Introspective Diffusion
                                  Language Models" summary page, serving section) */
  int32_t tile_k;              /* keys per k-tile; 0 -> 64 */
  uint32_t flags;              /* BCP_F_CHECK | BCP_F_LIVE_IN_CACHE */
  int32_t window;              /* sliding window W >= 1 in positions, or 0 for none: key
                                  position pk stays visible to query position pq only if
                                  pq - pk < W ("Inference: Fewer, smaller forwards", Advancement
                                  11); in mode A committed row j is at position j and live row i
                                  at kv_len + i, in mode B q_pos/kv_pos give them; tiles entirely
                                  outside the window are SKIP */
  const int32_t* q_pos;        /* [total_q] position of each live row; mode B with a window only */
  const int32_t* kv_pos;       /* [num_pages*page_size] position of each cache slot, beside
                                  kv_blk; mode B with a window only (committed with an id-only
                                  kv_commit_block, src_blk = q_pos, kv_blk_out = kv_pos) */
} bcp_meta;

/* Number of query tiles / key tiles of the step's tile grid (after the tile defaults).
 * nqt = ceil(max_q_len/tile_q); nkt = ceil(max_kv_len/tile_k) + ceil(max_q_len/tile_k):
 * the cached key tiles come first, then the live key tiles. Returns 0 on a bad meta. */
int32_t bcp_num_q_tiles(const bcp_meta* m);
int32_t bcp_num_k_tiles(const bcp_meta* m);

/* Device bytes of the step plan that build_tile_mask writes and attn_block_causal_paged
 * reads (0 on a bad meta). */
size_t bcp_plan_size(const bcp_meta* m);

/*
 * build_tile_mask -- classify every (query tile, key tile) pair of every sequence
 * ("FlexAttention with Aligned Tiles": a tile is fully included, fully excluded or
 * partially included; included tiles need no masking, excluded tiles no work).
 * A tile is SKIP if no in-range row sees any of its columns, FULL if every in-range row
 * sees all tile_k columns (a column past its region's length counts as not visible), and
 * PARTIAL otherwise. Computed from block-id ranges: SKIP iff (no valid row or column) or
 * min key block > max query block; FULL iff max key block <= min query block and all
 * tile_k columns are valid. Committed rows in mode A count as block -infinity.
 *
 *   tile_class  [batch, nqt, nkt] uint8 BCP_TILE_* codes, or NULL.
 *   phys_page   [batch, ceil(max_kv_len/tile_k), max(1, tile_k/page_size)] int32, or NULL:
 *               the physical page holding row t*tile_k + u*page_size of sequence s (the page
 *               table applied to the tile grid), -1 at or past kv_len[s]. When
 *               page_size > tile_k there is one entry per tile: the page of its first row.
 *   plan        [bcp_plan_size(m) bytes], or NULL: the step plan for attn_block_causal_paged
 *               (per q-tile list of non-skipped key tiles and a balanced split-KV work
 *               list). Only valid for the attention tile sizes (tile_q = the default,
 *               tile_k = 64) and only for metadata identical to the attention call's.
 * At least one output must be non-NULL. Errors: BCP_E_ARG, BCP_E_WORKSPACE (plan_bytes too
 * small), BCP_E_RANGE (checked mode), BCP_E_HIP.
 */
int build_tile_mask(const bcp_meta* m, uint8_t* tile_class, int32_t* phys_page, void* plan,
                    size_t plan_bytes, hipStream_t stream);

/* Device workspace bytes attn_block_causal_paged needs: the split-KV partial results, and
 * room to build the plan itself when it is called with plan == NULL. */
size_t attn_block_causal_paged_workspace_size(const bcp_meta* m);

/*
 * attn_block_causal_paged -- block-causal attention of the live rows over the paged cache
 * and the live rows themselves (definition at the top of this file).
 *   q, k_new, v_new, k_cache, v_cache: layouts above, dtype m->dtype; with
 *               BCP_F_LIVE_IN_CACHE the live keys and values are read from the caches at
 *               logical rows kv_len[s] + i and k_new/v_new are ignored (may be NULL).
 *   plan        from build_tile_mask with the same meta, or NULL (then it is built in the
 *               workspace first, costing two extra kernel launches).
 *   scale       softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   out         [total_q, Hq, d] dtype m->dtype (bf16 rounded to nearest even).
 *   lse         [total_q, Hq] float32 natural-log sum of exp of the scaled visible scores,
 *               or NULL.
 *   workspace   >= attn_block_causal_paged_workspace_size(m) bytes (need not be zeroed).
 *   stats       uint64[4] or NULL: counters incremented by this call -- FULL tiles
 *               computed, PARTIAL tiles computed, SKIP tiles not loaded (each per kv head),
 *               K/V bytes loaded.
 * Supported: head_dim 64/128; bf16 (MFMA path: 256 packed query rows per work item, or 64
 * for the narrow default) or f32 (vector path); tile_q and tile_k must equal their defaults. Every row must see at least one key (always true: a live row
 * sees itself); a row that sees none gets out = 0 and lse = -inf.
 * Errors: BCP_E_ARG, BCP_E_UNSUPPORTED, BCP_E_WORKSPACE, BCP_E_RANGE (checked), BCP_E_HIP.
 */
int attn_block_causal_paged(const bcp_meta* m, const void* q, const void* k_new,
                            const void* v_new, const void* k_cache, const void* v_cache,
                            const void* plan, float scale, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, uint64_t* stats,
                            hipStream_t stream);

/*
 * attn_block_causal_paged_noalloc -- attn_block_causal_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that forbid hipMalloc,
 * harnesses that forbid allocation): the same computation and kernels, bit for bit, but no
 * workspace argument. Its split-KV partial results (and the plan, when plan is NULL) live in
 * a static device array of BCP_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * GPU it runs on until the process ends; the call itself allocates nothing. Every call on a
 * GPU shares that GPU's array, so calls on one GPU that overlap in time (on different
 * streams, say) race: issue them on one stream, or use attn_block_causal_paged with a
 * workspace each. The array keeps whatever the last call left; nothing in it needs to start
 * at zero. The first call on a device looks up that device's copy (hipGetSymbolAddress).
 * Errors: as attn_block_causal_paged, and BCP_E_WORKSPACE when the step needs more scratch
 * than the array holds (64.5 MiB of partial results at head_dim 128, plus the plan when it
 * is NULL; a plan from build_tile_mask keeps any step within the limit).
 */
#define BCP_NOALLOC_SCRATCH_BYTES (76u << 20)
int attn_block_causal_paged_noalloc(const bcp_meta* m, const void* q, const void* k_new,
                                    const void* v_new, const void* k_cache, const void* v_cache,
                                    const void* plan, float scale, void* out, float* lse,
                                    uint64_t* stats, hipStream_t stream);

/*
 * kv_commit_block -- write finished rows into their cache pages ("KV Cache", step 3: a
 * block's keys and values are written to the cache by a separate pass once the block is
 * decided; "Fewer, smaller forwards", Advancement 11: arena entries carry their position
 * tag, here the block id).
 * For sequence s and r < cu_src[s+1]-cu_src[s]: source row
 *   row = src_row ? src_row[cu_src[s]+r] : cu_src[s]+r
 * is copied bit for bit from k_src/v_src [n_src, Hkv, d] to logical row dst_start[s]+r of
 * sequence s, i.e. page page_table[s, (dst_start[s]+r)/P], slot (dst_start[s]+r)%P, of
 * k_cache/v_cache; kv_blk_out[page*P+slot] = src_blk[row] when both are non-NULL. Every
 * other byte of the caches is left as it was. The caller maps the pages beforehand and
 * advances kv_len afterwards; the library never changes metadata.
 *   cu_src [batch+1], src_row [total_commit] or NULL, dst_start [batch],
 *   src_blk [n_src] or NULL, kv_blk_out [num_pages*P] or NULL.
 *   total_commit = host copy of cu_src[batch]; n_src = rows in k_src/v_src.
 * With k_src = v_src = NULL only the int32 tags move: kv_blk_out[page*P+slot] = src_blk[row]
 * (nothing at all when both are NULL). That commits rows whose keys and values already sit
 * in their slots (BCP_F_LIVE_IN_CACHE; in mode A committing them is then the caller's
 * kv_len update), and it commits position tags (src_blk = q_pos, kv_blk_out = kv_pos).
 * Two rows with the same destination slot race (checked mode rejects it with BCP_E_RANGE).
 * Uses m's dtype, batch, Hkv, head_dim, page_table, num_pages, page_size,
 * max_pages_per_seq and flags.
 */
int kv_commit_block(const bcp_meta* m, const void* k_src, const void* v_src,
                    const int32_t* cu_src, const int32_t* src_row, const int32_t* dst_start,
                    const int32_t* src_blk, int32_t total_commit, int32_t n_src,
                    void* k_cache, void* v_cache, int32_t* kv_blk_out, hipStream_t stream);

/*
 * Step graphs -- capture the calls a step makes on one stream and replay them
 * ("Inference for Interpretable Text-Diffusion Models", section "Making CDE Fast", Compilation
 * Strategy: fixed-shape decode graphs cut call latency; the Introspective Diffusion Language
 * Models summary page, serving implementation and ablation: the extend forward is captured
 * and replayed as a graph, the largest single gain in its system ablation).
 *   bcp_graph_begin(stream)        starts capturing `stream` (thread-local capture mode); the
 *                                  stream must not be the legacy default stream.
 *   bcp_graph_end(stream, &graph)  ends the capture and instantiates it; *graph is owned by
 *                                  the caller until bcp_graph_destroy.
 *   bcp_graph_launch(graph, stream) enqueues one replay on `stream`.
 *   bcp_graph_destroy(graph)       releases it (NULL is allowed).
 * Between begin and end, entry points enqueue their kernels into the capture instead of
 * running them; checked mode is refused there (BCP_E_ARG), since it copies to the host.
 * A replay reads the current contents of every buffer the captured calls named, so those
 * buffers must stay allocated, and the step's shapes (the host arguments) fixed, for as
 * long as the graph is replayed. The HIP runtime may allocate memory to instantiate a
 * graph; these are the only entry points that keep state past a call.
 * Errors: BCP_E_ARG (NULL graph pointer), BCP_E_HIP (the HIP graph call failed).
 */
typedef struct bcp_graph bcp_graph;
int bcp_graph_begin(hipStream_t stream);
int bcp_graph_end(hipStream_t stream, bcp_graph** graph);
int bcp_graph_launch(bcp_graph* graph, hipStream_t stream);
void bcp_graph_destroy(bcp_graph* graph);

/* Thread-local description of the last non-OK return on this thread (host string). */
const char* bcp_last_error(void);

/* BCP_ABI_VERSION of the loaded library. */
int bcp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BCP_H */
