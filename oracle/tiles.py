"""Tile classes of the block-causal mask, by brute force (oracle; test infrastructure only).

"Inference for Interpretable Text-Diffusion Models", section "FlexAttention with Aligned
Tiles" and the BlockMask tile figure: the mask is cut into tiles, each fully included
(no masking needed), fully excluded (no attention work at all) or partially included.

Grid convention: for sequence s, q-tile r covers live rows [r*tile_q, (r+1)*tile_q) and
rows at or past q_len are ignored. The key tiles are the ceil(max_kv_len/tile_k)
cached tiles (columns [t*tile_k, (t+1)*tile_k) of the committed rows) followed by the
ceil(max_q_len/tile_k) live tiles (same, over the live rows). A column at or past its
region's length counts as not visible. A tile is FULL if every in-range row sees every
one of its tile_k columns, SKIP if no in-range row sees any column (or it has no rows),
PARTIAL otherwise. This reads the classes off the dense mask; it does not use any
min/max shortcut.
"""
import numpy as np

from .mask import dense_mask
from .paging import translate

TILE_SKIP, TILE_PARTIAL, TILE_FULL = 0, 1, 2


def _ceil_div(a, b):
    return -(-int(a) // int(b))


def tile_classes(cu_q, kv_len, tile_q, tile_k, max_q_len, max_kv_len, block_size=None,
                 q_blk=None, kv_blk=None, page_table=None, page_size=None, num_pages=None,
                 window=None, q_pos=None, kv_pos=None):
    """uint8 [batch, nqt, nct + nlt] of TILE_* codes."""
    batch = len(cu_q) - 1
    tq, tk = int(tile_q), int(tile_k)
    nqt = _ceil_div(max_q_len, tq)
    nct, nlt = _ceil_div(max_kv_len, tk), _ceil_div(max_q_len, tk)
    out = np.zeros((batch, nqt, nct + nlt), dtype=np.uint8)
    for s in range(batch):
        lo, hi = int(cu_q[s]), int(cu_q[s + 1])
        q_len, n_cached = hi - lo, int(kv_len[s])
        if q_blk is not None:
            page, slot = translate(page_table, kv_len, page_size, num_pages, s)
            kb = np.asarray(kv_blk).reshape(-1)[page * int(page_size) + slot]
            qp = kp = None
            if window:
                qp = np.asarray(q_pos)[lo:hi]
                kp = np.asarray(kv_pos).reshape(-1)[page * int(page_size) + slot]
            M = dense_mask(q_len, n_cached, q_blk=np.asarray(q_blk)[lo:hi], kv_blk=kb, window=window,
                           q_pos=qp, kv_pos=kp)
        else:
            M = dense_mask(q_len, n_cached, block_size=block_size, window=window)
        # Pad each region's columns with "not visible" out to its whole tile grid.
        cached = np.zeros((q_len, nct * tk), dtype=bool)
        cached[:, :n_cached] = M[:, :n_cached]
        live = np.zeros((q_len, nlt * tk), dtype=bool)
        live[:, :q_len] = M[:, n_cached:]
        grid = np.concatenate([cached, live], axis=1).reshape(q_len, nct + nlt, tk)
        for r in range(nqt):
            sub = grid[r * tq:min((r + 1) * tq, q_len)]        # in-range rows only
            if sub.shape[0] == 0:
                continue                                         # stays SKIP
            anyv = sub.any(axis=(0, 2))
            allv = sub.all(axis=(0, 2))
            out[s, r] = np.where(allv, TILE_FULL, np.where(anyv, TILE_PARTIAL, TILE_SKIP))
    return out
