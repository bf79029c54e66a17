"""KV commit: finished rows written into their cache pages (oracle; test infrastructure only).

"Inference for Interpretable Text-Diffusion Models", section "KV Cache" (steps 1 and 3):
prefill stores the prompt's blocks in the cache, and a decoded block's keys and values
are stored by a pass of their own once none of its positions is still undecided. The
cache is paged (section "Paged Attention"), so logical destination row j of sequence s is page
page_table[s, j // P], slot j % P. Entries in the multi-canvas arena also record their
position tag beside the key and value ("Inference: Fewer, smaller forwards",
Advancement 11); here the tags are the block id and, for sliding-window layers, the
absolute position, each copied from its source row.

The copy is bitwise: every byte outside the destination slots keeps its old value. Two
rows landing on the same slot is an error (the result would depend on write order).
"""
import numpy as np

from .paging import translate


def _as_bits(a):
    a = np.asarray(a)
    if a.dtype == np.uint16 or a.dtype == np.uint32:
        return a
    if a.dtype == np.float32:
        return a.view(np.uint32)
    raise TypeError(f"unsupported stored dtype {a.dtype}")


def commit(k_cache, v_cache, k_src, v_src, cu_src, dst_start, page_table, page_size, num_pages,
           src_row=None, kv_blk=None, src_blk=None, kv_pos=None, src_pos=None):
    """Return (k_cache', v_cache', kv_blk') -- and kv_pos' as a fourth item when kv_pos is
    given -- after committing rows; inputs are not modified.

    For sequence s and r < cu_src[s+1]-cu_src[s]: source row = src_row[cu_src[s]+r]
    (identity when src_row is None) goes to logical row dst_start[s] + r.
    """
    kc, vc = _as_bits(k_cache).copy(), _as_bits(v_cache).copy()
    ks, vs = _as_bits(k_src), _as_bits(v_src)
    kb = None if kv_blk is None else np.asarray(kv_blk, dtype=np.int32).reshape(-1).copy()
    if src_blk is not None and kb is None:
        raise ValueError("src_blk given without kv_blk")
    kp = None if kv_pos is None else np.asarray(kv_pos, dtype=np.int32).reshape(-1).copy()
    if src_pos is not None and kp is None:
        raise ValueError("src_pos given without kv_pos")
    P = int(page_size)
    batch = len(cu_src) - 1
    seen = set()
    for s in range(batch):
        a, b = int(cu_src[s]), int(cu_src[s + 1])
        n = b - a
        if n < 0:
            raise ValueError("cu_src must be non-decreasing")
        if n == 0:
            continue
        dst = int(dst_start[s]) + np.arange(n, dtype=np.int64)
        page, slot = translate(page_table, np.full(batch, 0), P, num_pages, s, rows=dst)
        for r in range(n):
            row = a + r if src_row is None else int(src_row[a + r])
            if row < 0 or row >= ks.shape[0]:
                raise ValueError("source row out of range")
            key = (int(page[r]), int(slot[r]))
            if key in seen:
                raise ValueError(f"two rows commit to page {key[0]} slot {key[1]}")
            seen.add(key)
            kc[key] = ks[row]
            vc[key] = vs[row]
            if src_blk is not None:
                kb[key[0] * P + key[1]] = int(src_blk[row])
            if src_pos is not None:
                kp[key[0] * P + key[1]] = int(src_pos[row])
    if np.asarray(k_cache).dtype == np.float32:
        kc, vc = kc.view(np.float32), vc.view(np.float32)
    if kv_pos is not None:
        return kc, vc, kb, kp
    return kc, vc, kb
