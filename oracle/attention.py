"""Block-causal softmax attention over a paged cache, in float64 (oracle; test infrastructure only).

Definition (plain, dense): for sequence s and query head h, with kv head
g = h // (Hq / Hkv) (grouped-query attention: consecutive query heads share a kv head),
the keys are the committed rows gathered from their pages followed by the live rows of
the active blocks, and

    S = scale * q_h . K_g^T,   S = -inf where the block-causal mask forbids the pair,
    m = max_j S,  w = exp(S - m),  l = sum_j w,  O = (w . V_g) / l,  LSE = m + ln l.

The mask is mask.dense_mask (sections cited there, including the optional sliding
window); the gather is paging.gather. A row
with no visible key (impossible on valid input, since every row sees itself) gets O = 0
and LSE = -inf. The default scale is 1/sqrt(head_dim): the pages never state a scale,
and this is the usual one.
"""
import numpy as np

from .mask import dense_mask
from .numerics import widen
from .paging import translate


def attention_rows(q, k_new, v_new, k_cache, v_cache, cu_q, kv_len, page_table, page_size,
                   num_pages, s, rows=None, block_size=None, scale=None, q_blk=None, kv_blk=None,
                   row_chunk=512, window=None, q_pos=None, kv_pos=None):
    """O [len(rows), Hq, d] and LSE [len(rows), Hq] (float64) for local live rows of sequence s."""
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k_new.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    lo, hi = int(cu_q[s]), int(cu_q[s + 1])
    q_len, n_cached = hi - lo, int(kv_len[s])
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)

    page, slot = translate(page_table, kv_len, page_size, num_pages, s)
    Kf = np.concatenate([widen(k_cache[page, slot]), widen(k_new[lo:hi])], axis=0)  # [n, Hkv, d]
    Vf = np.concatenate([widen(v_cache[page, slot]), widen(v_new[lo:hi])], axis=0)
    if q_blk is not None:
        kb = np.asarray(kv_blk).reshape(-1)[page * int(page_size) + slot]
        qp = kp = None
        if window:
            qp = np.asarray(q_pos)[lo:hi]
            kp = np.asarray(kv_pos).reshape(-1)[page * int(page_size) + slot]
        M_all = dense_mask(q_len, n_cached, q_blk=np.asarray(q_blk)[lo:hi], kv_blk=kb, window=window,
                           q_pos=qp, kv_pos=kp)
    else:
        M_all = dense_mask(q_len, n_cached, block_size=block_size, window=window)

    O = np.zeros((rows.size, Hq, d), dtype=np.float64)
    L = np.full((rows.size, Hq), -np.inf, dtype=np.float64)
    for c0 in range(0, rows.size, row_chunk):
        r = rows[c0:c0 + row_chunk]
        M = M_all[r]                                  # [r, n]
        Q = widen(q[lo + r])                          # [r, Hq, d]
        for g in range(Hkv):
            Qg = Q[:, g * G:(g + 1) * G, :]           # [r, G, d]
            S = scale * (Qg.reshape(-1, d) @ Kf[:, g, :].T).reshape(r.size, G, -1)
            S = np.where(M[:, None, :], S, -np.inf)
            m = S.max(axis=2)                         # [r, G]
            ok = np.isfinite(m)
            m_safe = np.where(ok, m, 0.0)
            w = np.exp(S - m_safe[:, :, None])
            l = w.sum(axis=2)
            Og = (w.reshape(-1, w.shape[2]) @ Vf[:, g, :]).reshape(r.size, G, d)
            with np.errstate(invalid="ignore", divide="ignore"):
                Og = np.where(ok[:, :, None], Og / l[:, :, None], 0.0)
                Lg = np.where(ok, m_safe + np.log(l), -np.inf)
            O[c0:c0 + r.size, g * G:(g + 1) * G, :] = Og
            L[c0:c0 + r.size, g * G:(g + 1) * G] = Lg
    return O, L


def attention(q, k_new, v_new, k_cache, v_cache, cu_q, kv_len, page_table, page_size, num_pages,
              block_size=None, scale=None, q_blk=None, kv_blk=None, rows=None, window=None,
              q_pos=None, kv_pos=None):
    """O [total_q, Hq, d], LSE [total_q, Hq] in float64 for every sequence.

    rows: optional {s: local row indices} to compute a sample; other rows stay NaN.
    """
    total_q, Hq, d = q.shape
    O = np.full((total_q, Hq, d), np.nan, dtype=np.float64)
    L = np.full((total_q, Hq), np.nan, dtype=np.float64)
    batch = len(cu_q) - 1
    for s in range(batch):
        if rows is not None and s not in rows:
            continue
        r = None if rows is None else np.asarray(rows[s], dtype=np.int64)
        Os, Ls = attention_rows(q, k_new, v_new, k_cache, v_cache, cu_q, kv_len, page_table,
                                page_size, num_pages, s, rows=r, block_size=block_size,
                                scale=scale, q_blk=q_blk, kv_blk=kv_blk, window=window, q_pos=q_pos,
                                kv_pos=kv_pos)
        idx = int(cu_q[s]) + (np.arange(int(cu_q[s + 1]) - int(cu_q[s])) if r is None else r)
        O[idx] = Os
        L[idx] = Ls
    return O, L
