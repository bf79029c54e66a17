"""Dense block-causal visibility (oracle; test infrastructure only).

Columns are the kv_len committed rows of the sequence followed by its q_len live rows
(the active block or blocks, whose keys are passed in alongside the queries).

Mode A ("Inference for Interpretable Text-Diffusion Models", Background): the cache
holds only completed earlier blocks, so every committed row is visible; among live
rows, blocks of D consecutive rows counted from the sequence's first live row see
their own block and earlier ones: key j is visible to query i iff j//D <= i//D.

Mode B ("Inference: Fewer, smaller forwards", Advancement 1 and Advancement 11): every
row carries a block id (prompt, then canvas 1, 2, ...), committed entries carry theirs
beside the cache; a key is visible to a query iff the key's block id is not later than
the query's.

Sliding window ("Inference: Fewer, smaller forwards", Advancement 11: arena entries keep
their absolute position, so sliding-window layers can band-mask entries that fall outside
the window): with a window of W positions, a key at position pk stays visible to a query
at position pq only if pq - pk < W. Keys at later positions (inside the query's block)
are never cut by the window. Positions: in mode A the committed rows hold positions
0 .. kv_len-1 in order and live row i sits at kv_len + i; in mode B they are given per
row (q_pos) and per committed entry (kv_pos).
"""
import numpy as np


def dense_mask(q_len, kv_len, block_size=None, q_blk=None, kv_blk=None, window=None, q_pos=None,
               kv_pos=None):
    """Bool [q_len, kv_len + q_len]; q_blk [q_len] / kv_blk [kv_len] select mode B.

    window (>= 1) adds the sliding-window band; q_pos [q_len] / kv_pos [kv_len] give the
    positions in mode B (mode A derives them from the row order).
    """
    M = _block_mask(q_len, kv_len, block_size, q_blk, kv_blk)
    if not window:
        return M
    W = int(window)
    if W < 1:
        raise ValueError("window must be >= 1")
    q_len, kv_len = int(q_len), int(kv_len)
    if q_blk is None:
        if q_pos is not None or kv_pos is not None:
            raise ValueError("mode A derives positions from the row order")
        qp = kv_len + np.arange(q_len, dtype=np.int64)
        kp = np.arange(kv_len + q_len, dtype=np.int64)
    else:
        if q_pos is None or kv_pos is None:
            raise ValueError("a window in mode B needs q_pos and kv_pos")
        qp = np.asarray(q_pos, dtype=np.int64)
        kp = np.concatenate([np.asarray(kv_pos, dtype=np.int64), qp])
        if qp.size != q_len or kp.size != kv_len + q_len:
            raise ValueError("position arrays do not match the row counts")
    return M & ((qp[:, None] - kp[None, :]) < W)


def _block_mask(q_len, kv_len, block_size, q_blk, kv_blk):
    q_len, kv_len = int(q_len), int(kv_len)
    M = np.zeros((q_len, kv_len + q_len), dtype=bool)
    i = np.arange(q_len)
    if q_blk is None and kv_blk is None:
        D = int(block_size)
        if D < 1:
            raise ValueError("block size must be >= 1")
        M[:, :kv_len] = True
        M[:, kv_len:] = (i[None, :] // D) <= (i[:, None] // D)
        return M
    if q_blk is None or kv_blk is None:
        raise ValueError("mode B needs both q_blk and kv_blk")
    qb = np.asarray(q_blk, dtype=np.int64)
    kb = np.asarray(kv_blk, dtype=np.int64)
    if qb.size != q_len or kb.size != kv_len:
        raise ValueError("block-id arrays do not match the row counts")
    M[:, :kv_len] = kb[None, :] <= qb[:, None]
    M[:, kv_len:] = qb[None, :] <= qb[:, None]
    return M
