"""Small helpers the tests share: running the oracle on a workloads.Case, SDPA references.

Nothing here reimplements the oracle: hand placement of contiguous rows into pages is
test-fixture code, and SDPA is torch's own float64 CPU routine.
"""
import numpy as np
import torch

import oracle


def oracle_attention(case, rows=None, scale=None, window=None, q_pos=None, kv_pos=None):
    return oracle.attention(case.q, case.k_new, case.v_new, case.k_cache, case.v_cache, case.cu_q,
                            case.kv_len, case.page_table, case.page_size, case.num_pages,
                            block_size=case.block_size, scale=scale, q_blk=case.q_blk,
                            kv_blk=case.kv_blk, rows=rows, window=window, q_pos=q_pos, kv_pos=kv_pos)


def oracle_tiles(case, tile_q, tile_k, window=None, q_pos=None, kv_pos=None):
    return oracle.tile_classes(case.cu_q, case.kv_len, tile_q, tile_k, case.max_q_len,
                               case.max_kv_len, block_size=case.block_size, q_blk=case.q_blk,
                               kv_blk=case.kv_blk, page_table=case.page_table,
                               page_size=case.page_size, num_pages=case.num_pages, window=window,
                               q_pos=q_pos, kv_pos=kv_pos)


def sdpa64(q, k, v, causal=False, mask=None, scale=None):
    """torch SDPA in float64 on the CPU. q [Lq, H, d], k/v [Lk, H, d] (already expanded)."""
    tq = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).permute(1, 0, 2)[None]
    m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=bool))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, is_causal=causal,
                                                         scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def place_rows(rows_per_seq, page_table, page_size, num_pages, fill=np.nan):
    """Fixture: put each sequence's contiguous rows [n, H, d] into a fresh paged pool."""
    H, d = rows_per_seq[0].shape[1:]
    pool = np.full((num_pages, page_size, H, d), fill, dtype=np.float32)
    for s, rows in enumerate(rows_per_seq):
        for j in range(rows.shape[0]):
            pool[page_table[s][j // page_size], j % page_size] = rows[j]
    return pool


def expand_gqa(x, group):
    """[n, Hkv, d] -> [n, Hkv*group, d] with each kv head repeated for its query heads."""
    return np.repeat(x, group, axis=1)
