"""Logical-to-physical page translation (oracle; test infrastructure only).

"Inference for Interpretable Text-Diffusion Models", section "Paged Attention": each
request's KV cache sits in fixed-size pages that need not be contiguous, and a page
table maps the logical layout onto the physical pages; the page asks for strict error
checking, so every out-of-range access here raises.

Logical row j of sequence s lives in page page_table[s, j // P] at slot j % P.
"""
import numpy as np


def translate(page_table, kv_len, page_size, num_pages, s, rows=None):
    """Physical (page, slot) of logical rows `rows` (default 0..kv_len[s]-1) of sequence s."""
    page_table = np.asarray(page_table)
    P = int(page_size)
    n = int(kv_len[s])
    j = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if j.size == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    logical_page = j // P
    if logical_page.max() >= page_table.shape[1] or j.min() < 0:
        raise ValueError(f"sequence {s}: row beyond max_pages_per_seq*page_size")
    page = page_table[s, logical_page].astype(np.int64)
    if page.min() < 0 or page.max() >= num_pages:
        raise ValueError(f"sequence {s}: page id outside [0, {num_pages})")
    return page, j % P


def phys_page(page_table, kv_len, page_size, tile_k, n_cached_tiles):
    """Physical page of every page-sized piece of every cached key tile.

    Entry [s, t, u] is the page holding logical row t*tile_k + u*P, or -1 when that row
    is at or past kv_len[s]. When P > tile_k there is a single entry per tile: the page
    that contains the tile's first row.
    """
    page_table = np.asarray(page_table)
    P, Bk = int(page_size), int(tile_k)
    per_tile = max(1, Bk // P)
    B = page_table.shape[0]
    out = np.full((B, int(n_cached_tiles), per_tile), -1, dtype=np.int32)
    for s in range(B):
        for t in range(int(n_cached_tiles)):
            for u in range(per_tile):
                row = t * Bk + u * P
                if row < int(kv_len[s]):
                    out[s, t, u] = page_table[s, row // P]
    return out


def gather(pool, page_table, kv_len, page_size, num_pages, s):
    """Contiguous copy of sequence s's committed rows from a paged pool [pages, P, ...]."""
    page, slot = translate(page_table, kv_len, page_size, num_pages, s)
    return np.asarray(pool)[page, slot]
