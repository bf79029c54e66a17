"""Pins that fix the CPU oracle to facts from the pages and from mathematics.

Each test compares the oracle with something that is not the oracle: a value printed or
derived by hand (tests/golden), a closed form, a textbook or library routine (torch
SDPA in float64), an invariant the pages state, or brute force. They are chosen so a
dropped term, a wrong sign or index, an off-by-one in the mask or a transposed operand
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import TILE_FULL, TILE_PARTIAL, TILE_SKIP
from workloads import bf16_bits, config, make_case, multi_canvas_structure
from tests.oracle_helpers import expand_gqa, oracle_attention, oracle_tiles, place_rows, sdpa64

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
CODE = {"F": TILE_FULL, "P": TILE_PARTIAL, "S": TILE_SKIP}


def contiguous_case(rng, *, q_len, kv_len, Hq, Hkv, d, D, P, std=1.0, perm=True):
    """One sequence with contiguous logical K/V; placed into a permuted pool by the fixture."""
    npages = -(-(kv_len + q_len) // P) + 1
    pool_pages = npages + 3
    pages = rng.permutation(pool_pages)[:npages] if perm else np.arange(npages)
    pt = pages[None, :].astype(np.int32)
    Kc = (std * rng.standard_normal((kv_len, Hkv, d))).astype(np.float32)
    Vc = (std * rng.standard_normal((kv_len, Hkv, d))).astype(np.float32)
    q = (std * rng.standard_normal((q_len, Hq, d))).astype(np.float32)
    kn = (std * rng.standard_normal((q_len, Hkv, d))).astype(np.float32)
    vn = (std * rng.standard_normal((q_len, Hkv, d))).astype(np.float32)
    kc = place_rows([Kc], pt, P, pool_pages)
    vc = place_rows([Vc], pt, P, pool_pages)
    return dict(q=q, k_new=kn, v_new=vn, k_cache=kc, v_cache=vc, cu_q=np.array([0, q_len]),
                kv_len=np.array([kv_len]), page_table=pt, page_size=P, num_pages=pool_pages,
                block_size=D), (Kc, Vc)


def run(c, **kw):
    return oracle.attention(c["q"], c["k_new"], c["v_new"], c["k_cache"], c["v_cache"], c["cu_q"],
                            c["kv_len"], c["page_table"], c["page_size"], c["num_pages"],
                            block_size=c["block_size"], **kw)


# ---------------------------------------------------------------- numerics ----------

def test_widen_matches_torch_bfloat16():
    """bf16 bits widened by the oracle equal torch's own bfloat16 -> float64 conversion."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-8, 8, 4096)).astype(np.float32)
    bits = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.widen(bits), ref)


# ---------------------------------------------------------------- P1 / P2 / P3 -------

@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (8, 1)])
def test_D1_is_token_causal_attention(Hq, Hkv):
    """D=1 and an empty cache: block-causal = token-causal attention (SDPA is_causal).

    Block-causal with one token per block is ordinary causal attention; the causal
    extend of the introspective-diffusion serving stack is this case.
    """
    rng = np.random.default_rng(1)
    c, _ = contiguous_case(rng, q_len=37, kv_len=0, Hq=Hq, Hkv=Hkv, d=16, D=1, P=4)
    O, _ = run(c)
    ref = sdpa64(c["q"], expand_gqa(c["k_new"], Hq // Hkv), expand_gqa(c["v_new"], Hq // Hkv),
                 causal=True)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_D1_textbook_loop():
    """D=1 against a literal per-row loop of the softmax definition (3 rows, d=3)."""
    rng = np.random.default_rng(2)
    c, _ = contiguous_case(rng, q_len=3, kv_len=0, Hq=1, Hkv=1, d=3, D=1, P=2)
    O, L = run(c)
    q, k, v = (c[n].astype(np.float64)[:, 0] for n in ("q", "k_new", "v_new"))
    for i in range(3):
        s = [float(np.dot(q[i], k[j])) / math.sqrt(3) for j in range(i + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        o = [sum(w[j] * v[j][e] for j in range(i + 1)) / tot for e in range(3)]
        np.testing.assert_allclose(O[i, 0], o, atol=1e-13)
        assert abs(L[i, 0] - (mx + math.log(tot))) < 1e-13


@pytest.mark.parametrize("q_len,D", [(20, 20), (20, 64)])
def test_single_block_is_bidirectional(q_len, D):
    """D >= q_len with an empty cache: one block, full bidirectional attention."""
    rng = np.random.default_rng(3)
    c, _ = contiguous_case(rng, q_len=q_len, kv_len=0, Hq=4, Hkv=4, d=8, D=D, P=8)
    O, _ = run(c)
    np.testing.assert_allclose(O, sdpa64(c["q"], c["k_new"], c["v_new"]), atol=1e-12)


def test_decode_one_block_over_cache_is_unmasked_attention():
    """Mode-A decode of one block sees the whole cache plus its own block: unmasked SDPA
    over the contiguous [cached; live] keys (the fixture knows the contiguous rows)."""
    rng = np.random.default_rng(4)
    c, (Kc, Vc) = contiguous_case(rng, q_len=16, kv_len=45, Hq=4, Hkv=2, d=16, D=16, P=8)
    O, _ = run(c)
    K = np.concatenate([Kc, c["k_new"]]).astype(np.float64)
    V = np.concatenate([Vc, c["v_new"]]).astype(np.float64)
    np.testing.assert_allclose(O, sdpa64(c["q"], expand_gqa(K, 2), expand_gqa(V, 2)), atol=1e-12)


# ---------------------------------------------------------------- P4 hand cases -------

def _hand(D, kv_rows):
    g = GOLD["two_token_attention"]
    q = np.array(g["q"], np.float32)[:, None, :]
    k = np.array(g["k"], np.float32)[:, None, :]
    v = np.array(g["v"], np.float32)[:, None, :]
    if kv_rows == 0:
        pool = np.full((1, 1, 1, 2), np.nan, np.float32)
        return oracle.attention(q, k, v, pool, pool, [0, 2], [0], np.zeros((1, 1), np.int32), 1, 1,
                                block_size=D)
    # Row 0 committed into page 3 of a 4-page pool, row 1 live.
    pool_k = np.full((4, 1, 1, 2), np.nan, np.float32)
    pool_v = pool_k.copy()
    pool_k[3, 0] = k[0]
    pool_v[3, 0] = v[0]
    return oracle.attention(q[1:], k[1:], v[1:], pool_k, pool_v, [0, 1], [1],
                            np.array([[3, 0]], np.int32), 1, 4, block_size=D)


@pytest.mark.parametrize("which", ["D1", "D2", "decode"])
def test_hand_two_tokens(which):
    g = GOLD["two_token_attention"]
    O, L = _hand(1 if which == "D1" else 2, 1 if which == "decode" else 0)
    np.testing.assert_allclose(O[:, 0], g[which]["O"], atol=g["tol"])
    np.testing.assert_allclose(L[:, 0], g[which]["LSE"], atol=g["tol"])


def test_hand_two_tokens_closed_form():
    """Row 1 of D=1 in closed form: weights 1/(1+e^a), e^a/(1+e^a), a = 1/sqrt(2)."""
    a = 1 / math.sqrt(2)
    O, L = _hand(1, 0)
    assert abs(O[1, 0, 0] - 1 / (1 + math.exp(a))) < 1e-15
    assert abs(O[1, 0, 1] - math.exp(a) / (1 + math.exp(a))) < 1e-15
    assert abs(L[1, 0] - math.log(1 + math.exp(a))) < 1e-15


# ---------------------------------------------------------------- P5 mask readout -----

def _readout(q_len, kv_len, D=None, q_blk=None, kv_blk=None, P=2):
    """K = 0 gives equal weights over visible keys; one-hot V reads the mask out."""
    n = kv_len + q_len
    d = n
    eye = np.eye(n, dtype=np.float32)
    q = np.ones((q_len, 1, d), np.float32)
    kn = np.zeros((q_len, 1, d), np.float32)
    vn = eye[kv_len:, None, :]
    npg = max(1, -(-kv_len // P))
    pt = np.arange(npg, dtype=np.int32)[None, ::-1].copy()        # reversed pages
    kc = place_rows([np.zeros((kv_len, 1, d), np.float32)], pt, P, npg)
    vc = place_rows([eye[:kv_len, None, :]], pt, P, npg)
    kvb = None
    if kv_blk is not None:
        kvb = np.full(npg * P, -1, np.int32)
        for j, b in enumerate(kv_blk):
            kvb[pt[0, j // P] * P + j % P] = b
    O, _ = oracle.attention(q, kn, vn, kc, vc, [0, q_len], [kv_len], pt, P, npg, block_size=D,
                            q_blk=None if q_blk is None else np.asarray(q_blk, np.int32), kv_blk=kvb)
    return O[:, 0, :]


def test_mask_readout_mode_A():
    g = GOLD["mask_readout_D2"]
    vis = np.array(g["visible"], np.float64)
    O = _readout(g["q_len"], g["kv_len"], D=g["D"])
    np.testing.assert_allclose(O, vis / vis.sum(1, keepdims=True), atol=1e-15)


def test_mask_readout_mode_B():
    g = GOLD["mask_readout_canvases"]
    vis = np.array(g["visible"], np.float64)
    O = _readout(len(g["q_blk"]), len(g["kv_blk"]), q_blk=g["q_blk"], kv_blk=g["kv_blk"])
    np.testing.assert_allclose(O, vis / vis.sum(1, keepdims=True), atol=1e-15)


def test_zero_keys_give_mean_of_visible_values():
    """Closed form on the tiny workload shape: K = 0 -> O_i = mean of V over visible keys."""
    c1 = config(1)
    k0 = np.zeros_like(c1.k_new)
    kc0 = np.where(np.isnan(c1.k_cache), np.nan, 0.0).astype(np.float32)
    O, _ = oracle.attention(c1.q, k0, c1.v_new, kc0, c1.v_cache, c1.cu_q, c1.kv_len, c1.page_table,
                            c1.page_size, c1.num_pages, block_size=c1.block_size)
    V = np.concatenate([c1.v_cache[:3].reshape(48, 1, 64), c1.v_new]).astype(np.float64)
    # 48 committed rows plus one live block of D=16: every row sees all 64 keys.
    np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-12)


# ---------------------------------------------------------------- P6-P8 tiles ---------

def _prefill_tiles(tokens, D, tq, tk):
    return oracle.tile_classes([0, tokens], [0], tq, tk, tokens, 0, block_size=D)[0]


@pytest.mark.parametrize("key", ["figure_blockmask_tiles", "figure_prefill_blockmask"])
def test_page_figures_tile_classes(key):
    g = GOLD[key]
    got = _prefill_tiles(g["tokens"], g["D"], g["tile"], g["tile"])
    np.testing.assert_array_equal(got, [[CODE[x] for x in row] for row in g["classes"]])


def test_figure_blockmask_counts():
    got = _prefill_tiles(6, 2, 2, 2)
    assert (got == TILE_FULL).sum() == 6 and (got == TILE_SKIP).sum() == 3
    assert (got == TILE_PARTIAL).sum() == 0


def test_unaligned_tiles():
    g = GOLD["unaligned_tiles"]
    got = _prefill_tiles(g["tokens"], g["D"], g["tile_q"], g["tile_k"])
    np.testing.assert_array_equal(got, [[CODE[x] for x in row] for row in g["classes"]])


@pytest.mark.parametrize("tq,tk,full,partial", [(64, 64, 8256, 0), (128, 64, 4096, 64)])
def test_prefill_8192_tile_counts(tq, tk, full, partial):
    """8192-token prefill in blocks of 64: aligned tiles are all full or skipped; with
    128-row q-tiles each q-tile has one partial tile (its second block's own tile)."""
    got = _prefill_tiles(8192, 64, tq, tk)
    assert (got == TILE_FULL).sum() == full
    assert (got == TILE_PARTIAL).sum() == partial
    assert (got == TILE_SKIP).sum() == got.size - full - partial


def test_prefill_remainder_rule_and_commit_count():
    """Prefill figure: a 10-token prompt with D=4 commits floor(10/4)*4 = 8 rows (B0, B1);
    the 2 leftover prompt tokens stay in block B2 with 2 masked positions."""
    g = GOLD["figure_prefill_blockmask"]
    D, n = g["D"], g["prompt_tokens"]
    commit_rows = (n // D) * D
    assert commit_rows == g["cached_after_prefill"]
    assert n - commit_rows == g["next_block_fixed"]
    assert D - (n - commit_rows) == g["next_block_masked"]
    rng = np.random.default_rng(5)
    src = rng.standard_normal((n, 1, 2)).astype(np.float32)
    pool = np.full((3, D, 1, 2), np.nan, np.float32)
    kc, _, _ = oracle.commit(pool, pool, src, src, [0, commit_rows], [0],
                             np.array([[2, 0, 1]], np.int32), D, 3)
    assert np.isnan(kc.view(np.float32)[1]).all()                # third page untouched
    np.testing.assert_array_equal(kc.view(np.float32)[2], src[:4])
    np.testing.assert_array_equal(kc.view(np.float32)[0], src[4:8])


def _minmax_class(qb_rows, kb_cols, nvalid_cols, tk):
    """Independent formulation: SKIP iff min key block > max query block (or nothing valid);
    FULL iff max key block <= min query block and all tk columns valid; else PARTIAL."""
    if len(qb_rows) == 0 or nvalid_cols == 0:
        return TILE_SKIP
    if min(kb_cols) > max(qb_rows):
        return TILE_SKIP
    if max(kb_cols) <= min(qb_rows) and nvalid_cols == tk:
        return TILE_FULL
    return TILE_PARTIAL


@pytest.mark.parametrize("seed", range(6))
def test_tiles_brute_force_equals_minmax_rule(seed):
    """The brute-force classes equal a min/max-of-block-ids rule on random mode-B inputs
    (both orders of committed rows) and mode-A inputs with ragged lengths."""
    rng = np.random.default_rng(100 + seed)
    B = 3
    q_lens = rng.integers(0, 40, B)
    kv_lens = rng.integers(0, 50, B)
    tq, tk, P = [(8, 8, 4), (16, 8, 8), (4, 16, 4), (8, 4, 2), (32, 32, 16), (8, 16, 16)][seed]
    qb_seqs = [np.sort(rng.integers(1, 5, n)) for n in q_lens]
    kb_seqs = [rng.integers(0, 5, n) for n in kv_lens]
    c = make_case(seed, dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=4, block_size=3,
                  page_size=P, q_lens=q_lens, kv_lens=kv_lens, q_blk_seqs=qb_seqs,
                  kv_blk_seqs=kb_seqs, rng=rng)
    got = oracle_tiles(c, tq, tk)
    nct = -(-c.max_kv_len // tk)
    for s in range(B):
        for r in range(got.shape[1]):
            rows = qb_seqs[s][r * tq:(r + 1) * tq]
            for t in range(got.shape[2]):
                if t < nct:
                    cols = kb_seqs[s][t * tk:(t + 1) * tk]
                else:
                    u = t - nct
                    cols = qb_seqs[s][u * tk:(u + 1) * tk]
                assert got[s, r, t] == _minmax_class(list(rows), list(cols), len(cols), tk)
    # Mode A: committed rows act as block -inf, live row i as block i // D.
    c.q_blk = c.kv_blk = None
    got = oracle_tiles(c, tq, tk)
    for s in range(B):
        qa = [i // 3 for i in range(q_lens[s])]
        for r in range(got.shape[1]):
            rows = qa[r * tq:(r + 1) * tq]
            for t in range(got.shape[2]):
                if t < nct:
                    n = max(0, min(tk, int(kv_lens[s]) - t * tk))
                    cols = [-(10 ** 9)] * n
                else:
                    cols = qa[(t - nct) * tk:(t - nct + 1) * tk]
                assert got[s, r, t] == _minmax_class(rows, cols, len(cols), tk)


# ---------------------------------------------------------------- P9-P13 invariants ---

def test_page_permutation_invariance():
    """Relabelling physical pages (and the page table with them) changes nothing, exactly."""
    c = config(2)
    small = dict(rows={0: np.arange(0, 64, 9), 5: np.arange(3, 64, 11)})
    O1, L1 = oracle_attention(c, **small)
    rng = np.random.default_rng(7)
    perm = rng.permutation(c.num_pages)             # new page id of old page p = perm[p]
    inv = np.argsort(perm)
    c.k_cache, c.v_cache = c.k_cache[inv], c.v_cache[inv]
    c.page_table = np.where(c.page_table >= 0, perm[np.maximum(c.page_table, 0)], -1).astype(np.int32)
    O2, L2 = oracle_attention(c, **small)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_cached_row_order_invariance_mode_B():
    """Cache order may be compacted: permuting committed rows together with their block ids
    leaves every output unchanged (up to summation order)."""
    rng = np.random.default_rng(8)
    ql, kl, qb, kb, _, _ = multi_canvas_structure(rng, 2, 24, 16, 3)
    c1 = make_case(8, dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=1,
                   page_size=4, q_lens=ql, kv_lens=kl, q_blk_seqs=qb, kv_blk_seqs=kb,
                   rng=np.random.default_rng(9))
    O1, _ = oracle_attention(c1)
    # Rebuild sequence 1's cache with its committed rows in a random order.
    Kc = oracle.gather(c1.k_cache, c1.page_table, c1.kv_len, 4, c1.num_pages, 1)
    Vc = oracle.gather(c1.v_cache, c1.page_table, c1.kv_len, 4, c1.num_pages, 1)
    p = rng.permutation(kl[1])
    pt = c1.page_table
    kc, vc = c1.k_cache.copy(), c1.v_cache.copy()
    kvb = c1.kv_blk.copy()
    for j in range(kl[1]):
        page, slot = pt[1, j // 4], j % 4
        kc[page, slot], vc[page, slot] = Kc[p[j]], Vc[p[j]]
        kvb[page * 4 + slot] = kb[1][p[j]]
    c1.k_cache, c1.v_cache, c1.kv_blk = kc, vc, kvb
    O2, _ = oracle_attention(c1)
    np.testing.assert_allclose(O1, O2, atol=1e-12)


def test_multi_canvas_equals_prefix_attention():
    """Prefix attention: canvas i attends exactly to a contiguous prefix (prompt, earlier
    canvases, itself), so the multi-canvas output equals per-canvas unmasked SDPA over
    that prefix of committed and live rows."""
    rng = np.random.default_rng(10)
    ql, kl, qb, kb, live_pos, com_pos = multi_canvas_structure(rng, 3, 20, 12, 3)
    c = make_case(10, dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=1,
                  page_size=8, q_lens=ql, kv_lens=kl, q_blk_seqs=qb, kv_blk_seqs=kb,
                  rng=np.random.default_rng(11))
    O, _ = oracle_attention(c)
    for s in range(3):
        Kc = oracle.gather(c.k_cache, c.page_table, c.kv_len, 8, c.num_pages, s)
        Vc = oracle.gather(c.v_cache, c.page_table, c.kv_len, 8, c.num_pages, s)
        lo = c.cu_q[s]
        kbs, qbs = np.asarray(kb[s]), np.asarray(qb[s])
        for i in range(1, 4):
            rows = np.nonzero(qbs == i)[0]
            if rows.size == 0:
                continue
            K = np.concatenate([Kc[kbs <= i], c.k_new[lo + np.nonzero(qbs <= i)[0]]])
            V = np.concatenate([Vc[kbs <= i], c.v_new[lo + np.nonzero(qbs <= i)[0]]])
            ref = sdpa64(c.q[lo + rows], expand_gqa(K, 2), expand_gqa(V, 2))
            np.testing.assert_allclose(O[lo + rows], ref, atol=1e-12)


def test_prefix_invariance_of_completed_blocks():
    """A completed block's outputs do not change when later blocks are appended."""
    rng = np.random.default_rng(12)
    c, _ = contiguous_case(rng, q_len=40, kv_len=13, Hq=4, Hkv=1, d=16, D=8, P=4)
    O_all, L_all = run(c)
    for b in (1, 3):
        n = 8 * b
        cut = dict(c, q=c["q"][:n], k_new=c["k_new"][:n], v_new=c["v_new"][:n], cu_q=np.array([0, n]))
        O, L = run(cut)
        np.testing.assert_allclose(O, O_all[:n], atol=1e-12)
        np.testing.assert_allclose(L, L_all[:n], atol=1e-12)


@pytest.mark.parametrize("b", [1, 4])
def test_prefill_equals_commit_then_decode(b):
    """Cache equivalence: prefill of blocks 0..b equals committing blocks < b into pages
    and then decoding block b against the cache (the block-causal property that makes
    the cache valid)."""
    rng = np.random.default_rng(13)
    D, P, Hq, Hkv, d = 8, 4, 4, 2, 16
    n = D * (b + 1)
    c, _ = contiguous_case(rng, q_len=n, kv_len=0, Hq=Hq, Hkv=Hkv, d=d, D=D, P=P)
    O_pre, L_pre = run(c)
    # Commit rows [0, b*D) into a fresh permuted pool, then decode the last block.
    npool = n // P + 2
    pt = rng.permutation(npool)[None, : -(-n // P)].astype(np.int32)
    pool = np.full((npool, P, Hkv, d), np.nan, np.float32)
    kc, vc, _ = oracle.commit(pool, pool, c["k_new"], c["v_new"], [0, b * D], [0], pt, P, npool)
    kc, vc = kc.view(np.float32), vc.view(np.float32)
    sl = slice(b * D, n)
    O_dec, L_dec = oracle.attention(c["q"][sl], c["k_new"][sl], c["v_new"][sl], kc, vc, [0, D],
                                    [b * D], pt, P, npool, block_size=D)
    np.testing.assert_allclose(O_dec, O_pre[sl], atol=1e-12)
    np.testing.assert_allclose(L_dec, L_pre[sl], atol=1e-12)


# ---------------------------------------------------------------- P14 GQA, commit -----

def test_gqa_equals_mha_with_repeated_kv():
    """Grouped-query attention: query head h reads kv head h // G (consecutive groups);
    identical to multi-head attention on K/V repeated G times per head."""
    rng = np.random.default_rng(14)
    c, (Kc, Vc) = contiguous_case(rng, q_len=24, kv_len=19, Hq=8, Hkv=2, d=8, D=6, P=4)
    O, L = run(c)
    rep = dict(c, k_new=expand_gqa(c["k_new"], 4), v_new=expand_gqa(c["v_new"], 4),
               k_cache=expand_gqa(c["k_cache"].reshape(-1, 2, 8), 4).reshape(c["k_cache"].shape[:2] + (8, 8)),
               v_cache=expand_gqa(c["v_cache"].reshape(-1, 2, 8), 4).reshape(c["v_cache"].shape[:2] + (8, 8)))
    O2, L2 = run(rep)
    np.testing.assert_allclose(O, O2, atol=1e-14)
    np.testing.assert_allclose(L, L2, atol=1e-14)


def test_hand_commit_slots():
    g = GOLD["hand_commit"]
    P = g["page_size"]
    src = np.arange(1, 4, dtype=np.float32).reshape(3, 1, 1)
    pool = np.zeros((6, P, 1, 1), np.float32)
    kc, _, kvb = oracle.commit(pool, pool, src, src, [0, 3], [g["dst_start"]],
                               np.array([g["page_table"]], np.int32), P, 6,
                               kv_blk=np.full(12, -1, np.int32), src_blk=np.array([7, 8, 9]))
    kc = kc.view(np.float32)
    for r, (page, slot) in enumerate(g["slots"]):
        assert kc[page, slot, 0, 0] == r + 1
        assert kvb[page * P + slot] == 7 + r
    assert np.count_nonzero(kc) == 3 and np.count_nonzero(kvb >= 0) == 3


def test_commit_round_trip_and_untouched_bytes():
    """Commit then gather returns the source bits; every other byte keeps its pre-image."""
    rng = np.random.default_rng(15)
    P, Hkv, d, npool = 4, 2, 8, 16
    src = bf16_bits(rng.standard_normal((11, Hkv, d)).astype(np.float32))
    pool = np.full((npool, P, Hkv, d), 0x7FC0, np.uint16)
    pt = rng.permutation(npool)[:8].reshape(2, 4).astype(np.int32)
    src_row = np.array([10, 3, 4, 0, 1, 2, 5, 6, 7], np.int64)
    kc, vc, _ = oracle.commit(pool, pool, src, src, [0, 4, 9], [5, 2], pt, P, npool, src_row=src_row)
    got0 = oracle.gather(kc, pt, [9, 11], P, npool, 0)[5:9]
    got1 = oracle.gather(kc, pt, [9, 11], P, npool, 1)[2:7]
    np.testing.assert_array_equal(got0, src[src_row[:4]])
    np.testing.assert_array_equal(got1, src[src_row[4:]])
    assert (kc == 0x7FC0).sum() == pool.size - 9 * Hkv * d


def test_commit_rejects_duplicate_and_out_of_range():
    pool = np.zeros((2, 2, 1, 1), np.float32)
    src = np.ones((3, 1, 1), np.float32)
    with pytest.raises(ValueError):   # sequences 0 and 1 share page 1 slot 0
        oracle.commit(pool, pool, src, src, [0, 1, 2], [2, 0], np.array([[0, 1], [1, 0]], np.int32), 2, 2)
    with pytest.raises(ValueError):   # page id past the pool
        oracle.commit(pool, pool, src, src, [0, 1], [0], np.array([[5, 0]], np.int32), 2, 2)
    with pytest.raises(ValueError):   # row past max_pages_per_seq * P
        oracle.commit(pool, pool, src, src, [0, 1], [4], np.array([[0, 1]], np.int32), 2, 2)


def test_hand_phys_page():
    g = GOLD["hand_phys_page"]
    got = oracle.phys_page(np.array([g["page_table"]], np.int32), [g["kv_len"]], g["page_size"],
                           g["tile_k"], -(-g["kv_len"] // g["tile_k"]))
    np.testing.assert_array_equal(got[0], g["phys_page"])


def test_phys_page_large_pages():
    """Pages larger than a tile: one entry per tile, the page containing its first row."""
    got = oracle.phys_page(np.array([[9, 4]], np.int32), [70], 64, 16, 5)
    np.testing.assert_array_equal(got[0, :, 0], [9, 9, 9, 9, 4])


def test_translate_rejects_bad_pages():
    with pytest.raises(ValueError):
        oracle.translate(np.array([[0, -1]], np.int32), [3], 2, 4, 0)
    with pytest.raises(ValueError):
        oracle.translate(np.array([[0, 1]], np.int32), [5], 2, 4, 0)


# ---------------------------------------------------------------- stress ---------------

def test_large_scores_rescale_path():
    """Scores with a large spread and keys arranged so the running max grows row by row:
    the float64 definition still matches SDPA."""
    rng = np.random.default_rng(16)
    c, (Kc, Vc) = contiguous_case(rng, q_len=32, kv_len=70, Hq=2, Hkv=1, d=16, D=32, P=8, std=2.0)
    O, _ = run(c, scale=1.0)
    K = np.concatenate([Kc, c["k_new"]]).astype(np.float64)
    V = np.concatenate([Vc, c["v_new"]]).astype(np.float64)
    np.testing.assert_allclose(O, sdpa64(c["q"], expand_gqa(K, 2), expand_gqa(V, 2), scale=1.0),
                               atol=1e-11)


def test_score_shift_changes_only_the_lse():
    """Adding c*e0 to every key, cached and live, adds scale*c*q[i,h,0] to every score of
    query row (i, h): a constant per row, so the softmax is unchanged and the natural-log LSE
    moves by exactly that constant. With c = 1024 and inputs on a 1/64 grid the shifted keys
    are exact in float32, and the shifts (past 800 natural-log units, beyond where exp
    overflows or underflows even in float64) test the oracle's stability."""
    rng = np.random.default_rng(61)
    c, _ = contiguous_case(rng, q_len=40, kv_len=90, Hq=4, Hkv=2, d=16, D=16, P=8, std=2.0)
    for k in ("q", "k_new", "v_new", "k_cache", "v_cache"):
        c[k] = np.where(np.isfinite(c[k]), np.round(c[k] * 64) / 64, c[k]).astype(np.float32)
    O, L = run(c, scale=0.25)
    shifted = dict(c)
    shifted["k_new"] = c["k_new"].copy()
    shifted["k_new"][..., 0] += 1024.0
    shifted["k_cache"] = c["k_cache"].copy()
    shifted["k_cache"][..., 0] += 1024.0         # NaN slots stay NaN and are never read
    O2, L2 = run(shifted, scale=0.25)
    shift = 0.25 * 1024.0 * c["q"][..., 0].astype(np.float64)
    assert np.abs(shift).max() > 800             # exp overflows float64 past ~709
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-9)
    np.testing.assert_allclose(L2 - L, shift, rtol=0, atol=1e-9)


def test_workload_shapes():
    """The named workloads have the stated shapes (cheap structural checks)."""
    c1 = config(1)
    assert (c1.batch, c1.num_q_heads, c1.num_kv_heads, c1.head_dim) == (1, 2, 1, 64)
    assert c1.kv_len.tolist() == [48] and c1.q_lens.tolist() == [16]
    assert c1.page_table.tolist() == [[0, 1, 2, 3]] and c1.dtype == "f32"
    assert np.isnan(c1.k_cache[3]).all() and not np.isnan(c1.k_cache[:3]).any()


# ---------------------------------------------------------------- sliding window ----
# "Inference: Fewer, smaller forwards", Advancement 11: arena entries keep their absolute
# position, so a sliding-window layer can band-mask entries outside the window. Reading:
# a key at position pk is visible to a query at position pq only if pq - pk < W (and the
# block rule allows it); keys at later positions are never cut by the window.

def test_window_one_with_token_blocks_sees_only_itself():
    """W = 1, D = 1, empty cache: each row's only visible key is its own, so O = v_i and
    LSE = scale * q_i . k_i exactly (softmax over one key)."""
    rng = np.random.default_rng(71)
    c, _ = contiguous_case(rng, q_len=11, kv_len=0, Hq=2, Hkv=2, d=8, D=1, P=4)
    O, L = run(c, window=1)
    np.testing.assert_allclose(O, c["v_new"].astype(np.float64), rtol=0, atol=1e-15)
    lse = (c["q"].astype(np.float64) * c["k_new"].astype(np.float64)).sum(-1) / math.sqrt(8)
    np.testing.assert_allclose(L, lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("W", [1, 3, 7, 40])
def test_token_causal_window_equals_sdpa_on_key_slices(W):
    """D = 1 with a window: row i attends to keys max(0, i-W+1) .. i, which torch SDPA
    (float64, no mask) computes on that slice of the keys, row by row."""
    rng = np.random.default_rng(72)
    c, _ = contiguous_case(rng, q_len=23, kv_len=0, Hq=2, Hkv=1, d=8, D=1, P=4)
    O, _ = run(c, window=W)
    k, v = expand_gqa(c["k_new"], 2), expand_gqa(c["v_new"], 2)
    for i in range(23):
        a = max(0, i - W + 1)
        ref = sdpa64(c["q"][i:i + 1], k[a:i + 1], v[a:i + 1])
        np.testing.assert_allclose(O[i:i + 1], ref, atol=1e-12)


@pytest.mark.parametrize("W", [5, 30, 61])
def test_window_over_cache_equals_sdpa_on_position_slices(W):
    """One bidirectional block (D >= q_len) over a cache: row i at position kv_len + i sees
    the contiguous positions from kv_len + i - W + 1 on (cached then live), i.e. SDPA over
    that slice of the concatenated [cached; live] keys."""
    rng = np.random.default_rng(73)
    q_len, kv_len = 16, 45
    c, (Kc, Vc) = contiguous_case(rng, q_len=q_len, kv_len=kv_len, Hq=4, Hkv=2, d=16, D=16, P=8)
    O, _ = run(c, window=W)
    K = expand_gqa(np.concatenate([Kc, c["k_new"]]), 2)
    V = expand_gqa(np.concatenate([Vc, c["v_new"]]), 2)
    for i in range(q_len):
        a = max(0, kv_len + i - W + 1)
        np.testing.assert_allclose(O[i:i + 1], sdpa64(c["q"][i:i + 1], K[a:], V[a:]), atol=1e-12)


def test_window_wider_than_the_sequence_changes_nothing():
    rng = np.random.default_rng(74)
    c, _ = contiguous_case(rng, q_len=20, kv_len=33, Hq=4, Hkv=2, d=8, D=4, P=8)
    O0, L0 = run(c)
    O1, L1 = run(c, window=20 + 33)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(L0, L1)


def test_mode_B_positions_in_row_order_equal_mode_A_window():
    """Mode B with block ids and positions laid out as mode A has them implicitly
    (committed row j at position j and block -1; live row i at kv_len + i, block i // D)
    gives the same result as mode A with the same window."""
    rng = np.random.default_rng(75)
    q_len, kv_len, D, P, W = 19, 27, 4, 8, 9
    c, _ = contiguous_case(rng, q_len=q_len, kv_len=kv_len, Hq=2, Hkv=1, d=8, D=D, P=P)
    pt = c["page_table"][0]
    kv_blk = np.full(c["num_pages"] * P, 99, np.int32)
    kv_pos = np.full(c["num_pages"] * P, -10 ** 6, np.int32)
    for j in range(kv_len):
        kv_blk[pt[j // P] * P + j % P] = -1
        kv_pos[pt[j // P] * P + j % P] = j
    q_blk = (np.arange(q_len) // D).astype(np.int32)
    q_pos = (kv_len + np.arange(q_len)).astype(np.int32)
    OA, LA = run(c, window=W)
    OB, LB = run(c, window=W, q_blk=q_blk, kv_blk=kv_blk, q_pos=q_pos, kv_pos=kv_pos)
    np.testing.assert_array_equal(OA, OB)
    np.testing.assert_array_equal(LA, LB)


def _window_class_mode_A(i0, i1, j0, nvalid, tk, kvl, D, W, cached):
    """Class of a mode-A tile with a window, from interval bounds (rows i0..i1-1 of the
    q-tile, keys j0..j0+nvalid-1 of the region): for row i the visible keys form the
    interval [lo(i), hi(i)], both bounds non-decreasing in i."""
    if i1 <= i0 or nvalid <= 0:
        return TILE_SKIP
    jl = j0 + nvalid - 1
    if cached:   # position j; every committed row passes the block rule
        lo = lambda i: max(j0, kvl + i - W + 1)
        hi = lambda i: jl
    else:        # position kv_len + j; block rule j // D <= i // D
        lo = lambda i: max(j0, i - W + 1)
        hi = lambda i: min(jl, (i // D + 1) * D - 1)
    seen = [lo(i) <= hi(i) for i in range(i0, i1)]
    full = nvalid == tk and all(lo(i) == j0 and hi(i) == jl for i in range(i0, i1))
    return TILE_FULL if full else (TILE_PARTIAL if any(seen) else TILE_SKIP)


@pytest.mark.parametrize("seed", range(4))
def test_window_tiles_brute_force_equals_interval_rule(seed):
    """Mode-A tile classes with a window, read off the dense mask, equal the per-row
    interval rule above (which the kernels' classifier follows in closed form)."""
    rng = np.random.default_rng(200 + seed)
    B = 3
    q_lens = rng.integers(0, 70, B)
    kv_lens = rng.integers(0, 90, B)
    tq, tk, P, D, W = [(8, 8, 4, 3, 5), (16, 8, 8, 4, 17), (4, 16, 4, 1, 9), (32, 16, 16, 8, 40)][seed]
    c = make_case(seed, dtype="f32", num_q_heads=1, num_kv_heads=1, head_dim=4, block_size=D,
                  page_size=P, q_lens=q_lens, kv_lens=kv_lens, rng=rng)
    got = oracle.tile_classes(c.cu_q, c.kv_len, tq, tk, c.max_q_len, c.max_kv_len, block_size=D, window=W)
    nct = -(-c.max_kv_len // tk)
    for s in range(B):
        for r in range(got.shape[1]):
            i0, i1 = r * tq, min((r + 1) * tq, int(q_lens[s]))
            for t in range(got.shape[2]):
                cached = t < nct
                j0 = (t if cached else t - nct) * tk
                n = max(0, min(tk, (int(kv_lens[s]) if cached else int(q_lens[s])) - j0))
                assert got[s, r, t] == _window_class_mode_A(i0, i1, j0, n, tk, int(kv_lens[s]), D, W, cached)


def test_commit_copies_position_tags():
    """Commit writes each row's position beside its block id, at the row's slot only."""
    g = GOLD["hand_commit"]
    P = g["page_size"]
    src = np.arange(1, 4, dtype=np.float32).reshape(3, 1, 1)
    pool = np.zeros((6, P, 1, 1), np.float32)
    kc, _, kvb, kvp = oracle.commit(pool, pool, src, src, [0, 3], [g["dst_start"]],
                                    np.array([g["page_table"]], np.int32), P, 6,
                                    kv_blk=np.full(12, -1, np.int32), src_blk=np.array([7, 8, 9]),
                                    kv_pos=np.full(12, -1, np.int32), src_pos=np.array([40, 41, 42]))
    for r, (page, slot) in enumerate(g["slots"]):
        assert kvp[page * P + slot] == 40 + r
    assert np.count_nonzero(kvp >= 0) == 3


# ------------------------------------------------ row chunks and row sampling --------
# The oracle works through a sequence's live rows 512 at a time and can compute a chosen
# subset of rows. Both paths are pinned here against SDPA on inputs long enough to cross
# several chunk boundaries.

def test_rows_beyond_one_chunk_equal_sdpa_token_causal():
    """1100 token-causal rows (D=1, empty cache) -- three chunks of 512 -- against SDPA."""
    rng = np.random.default_rng(71)
    c, _ = contiguous_case(rng, q_len=1100, kv_len=0, Hq=4, Hkv=2, d=16, D=1, P=16)
    O, L = run(c)
    ref = sdpa64(c["q"], expand_gqa(c["k_new"], 2), expand_gqa(c["v_new"], 2), causal=True)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    # LSE of the first row (it sees only itself) is its own scaled score.
    q0, k0 = c["q"][0].astype(np.float64), expand_gqa(c["k_new"], 2)[0].astype(np.float64)
    np.testing.assert_allclose(L[0], (q0 * k0).sum(-1) / 4.0, rtol=0, atol=1e-12)


def block_causal_mask(q_len, kv_len, D):
    """Visibility written out per pair: cached keys always, live key j iff j // D <= i // D."""
    m = np.zeros((q_len, kv_len + q_len), dtype=bool)
    for i in range(q_len):
        m[i, :kv_len] = True
        for j in range(q_len):
            m[i, kv_len + j] = (j // D) <= (i // D)
    return m


def test_rows_beyond_one_chunk_equal_sdpa_block_causal_over_cache():
    """1030 live rows in blocks of 37 over a cache of 50 rows: the block edges fall at
    different offsets in each 512-row chunk; SDPA with the mask written out pair by pair."""
    rng = np.random.default_rng(72)
    q_len, kv_len, D = 1030, 50, 37
    c, (Kc, Vc) = contiguous_case(rng, q_len=q_len, kv_len=kv_len, Hq=2, Hkv=1, d=8, D=D, P=16)
    O, _ = run(c)
    K = expand_gqa(np.concatenate([Kc, c["k_new"]]), 2)
    V = expand_gqa(np.concatenate([Vc, c["v_new"]]), 2)
    ref = sdpa64(c["q"], K, V, mask=block_causal_mask(q_len, kv_len, D))
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_sampled_rows_equal_sdpa_and_the_full_call():
    """rows= computes exactly the chosen rows: against SDPA directly, and against the same
    rows of the full call (rows on both sides of each chunk edge, out of order, repeated)."""
    rng = np.random.default_rng(73)
    q_len, kv_len, D = 1100, 70, 64
    c, (Kc, Vc) = contiguous_case(rng, q_len=q_len, kv_len=kv_len, Hq=4, Hkv=1, d=16, D=D, P=8)
    rows = np.array([1099, 0, 511, 512, 513, 700, 1023, 1024, 5, 512])
    Os, Ls = oracle.attention_rows(c["q"], c["k_new"], c["v_new"], c["k_cache"], c["v_cache"], c["cu_q"],
                                   c["kv_len"], c["page_table"], c["page_size"], c["num_pages"], 0,
                                   rows=rows, block_size=D)
    K = expand_gqa(np.concatenate([Kc, c["k_new"]]), 4)
    V = expand_gqa(np.concatenate([Vc, c["v_new"]]), 4)
    ref = sdpa64(c["q"], K, V, mask=block_causal_mask(q_len, kv_len, D))
    np.testing.assert_allclose(Os, ref[rows], rtol=0, atol=1e-12)
    O, L = run(c)
    np.testing.assert_allclose(Os, O[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Ls, L[rows], rtol=0, atol=1e-12)
    # Through the batch wrapper: the sampled rows are filled, every other row stays NaN.
    Ob, _ = run(c, rows={0: rows})
    np.testing.assert_allclose(Ob[rows], ref[rows], rtol=0, atol=1e-12)
    others = np.setdiff1d(np.arange(q_len), rows)
    assert np.isnan(Ob[others]).all()
