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
"""
import numpy as np


def dense_mask(q_len, kv_len, block_size=None, q_blk=None, kv_blk=None):
    """Bool [q_len, kv_len + q_len]; q_blk [q_len] / kv_blk [kv_len] select mode B."""
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
