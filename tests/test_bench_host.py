"""Host-side checks of bench.py's accounting: the useful-FLOP count it prices the roofline
with equals the number of visible (row, key) pairs of the oracle's dense mask."""
import numpy as np
import pytest

import bench
import oracle
from workloads import make_case


def _dense_visible(case, window=None):
    n = 0
    for s in range(case.batch):
        ql, kl = int(case.q_lens[s]), int(case.kv_len[s])
        if case.q_blk is None:
            M = oracle.dense_mask(ql, kl, block_size=case.block_size, window=window)
        else:
            M = oracle.dense_mask(ql, kl, q_blk=case.q_blk_seqs[s], kv_blk=case.kv_blk_seqs[s])
        n += int(M.sum())
    return n


@pytest.mark.parametrize("window", [0, 1, 5, 40, 1000])
@pytest.mark.parametrize("D", [1, 4, 16])
def test_flop_count_matches_dense_mask_mode_A(window, D):
    rng = np.random.default_rng(100 + D)
    case = make_case(100 + D, dtype="bf16", num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=D,
                     page_size=8, q_lens=[1, 17, 40, 9], kv_lens=[0, 60, 3, 130], rng=rng)
    flops, cached_kv, _, _ = bench.workload_stats(case, window)
    assert flops == 4.0 * 64 * 4 * _dense_visible(case, window or None)
    # Committed rows any live row sees: all of them, or the last W-1 under a window.
    rows = sum(min(k, window - 1) if window else k for k in case.kv_len.tolist())
    assert cached_kv == rows * 1 * 64 * 2 * 2


def test_flop_count_matches_dense_mask_mode_B():
    rng = np.random.default_rng(7)
    q_lens, kv_lens = [5, 30, 12], [0, 44, 9]
    qb = [np.sort(rng.integers(1, 4, n)) for n in q_lens]
    kb = [np.sort(rng.integers(0, 4, n)) for n in kv_lens]
    case = make_case(7, dtype="bf16", num_q_heads=2, num_kv_heads=2, head_dim=64, block_size=1,
                     page_size=8, q_lens=q_lens, kv_lens=kv_lens, q_blk_seqs=qb, kv_blk_seqs=kb, rng=rng)
    flops, _, _, _ = bench.workload_stats(case)
    assert flops == 4.0 * 64 * 2 * _dense_visible(case)


def test_flop_count_matches_dense_mask_mode_B_window():
    from workloads import multi_canvas_structure, with_positions
    rng = np.random.default_rng(9)
    ql, kl, qb, kb, lp, cp = multi_canvas_structure(rng, 3, 30, 12, 3)
    case = with_positions(make_case(9, dtype="bf16", num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=1,
                                    page_size=8, q_lens=ql, kv_lens=kl, q_blk_seqs=qb, kv_blk_seqs=kb, rng=rng),
                          lp, cp)
    for W in (1, 7, 25):
        flops, _, _, _ = bench.workload_stats(case, W)
        n = 0
        for s in range(case.batch):
            lo, hi = int(case.cu_q[s]), int(case.cu_q[s + 1])
            n += int(oracle.dense_mask(hi - lo, int(case.kv_len[s]), q_blk=case.q_blk_seqs[s],
                                       kv_blk=case.kv_blk_seqs[s], window=W, q_pos=case.q_pos[lo:hi],
                                       kv_pos=np.asarray(cp[s])).sum())
        assert flops == 4.0 * 64 * 2 * n
