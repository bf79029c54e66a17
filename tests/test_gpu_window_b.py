"""GPU parity of the sliding window in mode B: block ids and absolute positions per entry.

"Inference: Fewer, smaller forwards", Advancement 11: arena entries keep their absolute
position, so sliding-window layers band-mask entries outside the window, and multi-canvas
decoding keeps going with more canvases. A key is visible to a live row iff its block id is
not later and its position lies fewer than W positions before the row's. Positions follow
the multi-canvas layout (prompt, then each canvas in order); committed slots carry them in
kv_pos beside kv_blk, live rows in q_pos.
"""
import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
import oracle
from tests.oracle_helpers import oracle_attention, oracle_tiles
from tests.test_gpu_parity import assert_close, say
from workloads import config, make_case, multi_canvas_structure, with_positions
from workloads.device import DeviceCase

pytestmark = pytest.mark.gpu


def canvas_case(seed, batch=3, prompt=40, canvas=24, n_canvas=3, G=4, Hkv=2, d=128, P=16, dtype="bf16",
                shuffle=False):
    """shuffle: the rows of each sequence in promotion order -- committed rows in random
    slot order and live rows interleaved across canvases, each with its id and position."""
    rng = np.random.default_rng(seed)
    ql, kl, qb, kb, live_pos, com_pos = multi_canvas_structure(rng, batch, prompt, canvas, n_canvas)
    if shuffle:
        for s in range(batch):
            p = rng.permutation(len(qb[s]))
            qb[s], live_pos[s] = [qb[s][i] for i in p], [live_pos[s][i] for i in p]
            p = rng.permutation(len(kb[s]))
            kb[s], com_pos[s] = [kb[s][i] for i in p], [com_pos[s][i] for i in p]
    case = make_case(seed, dtype=dtype, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d, block_size=1,
                     page_size=P, q_lens=ql, kv_lens=kl, q_blk_seqs=qb, kv_blk_seqs=kb,
                     qkv_std=1 / np.sqrt(d), rng=rng)
    return case, positions(case, live_pos, com_pos)


def positions(case, live_pos, com_pos):
    with_positions(case, live_pos, com_pos)
    return case.q_pos, case.kv_pos


def run(case, q_pos, kv_pos, window, plan=True, tile=None):
    dc = DeviceCase(case)
    qp = torch.from_numpy(q_pos).cuda()
    kp = torch.from_numpy(kv_pos).cuda()
    kw = dict(dc.meta_kwargs(), check=True, window=window, q_pos=qp, kv_pos=kp)
    meta = bcp.StepMeta(**kw)
    out = torch.full_like(dc.q, float("nan"))
    lse = torch.full(tuple(dc.q.shape[:2]), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    plan_t = None
    if plan:
        plan_t = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
        bcp.build_tile_mask(meta, plan=plan_t)
    bcp.attn_block_causal_paged(meta, dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, out, plan=plan_t,
                                lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return out, lse, (dc, qp, kp)


SMALL = [
    dict(seed=101, W=8),
    dict(seed=102, W=30, G=2, d=64, P=8),
    dict(seed=103, W=1),
    dict(seed=104, W=55, prompt=70, canvas=40, P=12),
    dict(seed=105, W=200, batch=4, prompt=300, canvas=64, n_canvas=4),       # wider than some sequences
    dict(seed=106, W=20, G=8, d=128, P=3),
    dict(seed=107, W=25, dtype="f32"),
    # narrow q-tiles (at most 64 packed rows per sequence and kv head): the narrow kernel
    dict(seed=108, W=12, G=4, Hkv=2, d=128, prompt=30, canvas=8, n_canvas=2, P=16, narrow=True),
    dict(seed=109, W=5, G=16, Hkv=1, d=64, prompt=20, canvas=2, n_canvas=2, P=8, narrow=True),
    # promotion order
    dict(seed=110, W=30, shuffle=True),
    dict(seed=115, W=200, batch=4, prompt=300, canvas=64, n_canvas=4, P=8, shuffle=True),
    dict(seed=116, W=9, G=4, Hkv=2, d=128, prompt=40, canvas=8, n_canvas=2, P=16, narrow=True, shuffle=True),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_mode_B_window_small(spec):
    spec = dict(spec)
    W = spec.pop("W")
    narrow = spec.pop("narrow", False)
    case, (q_pos, kv_pos) = canvas_case(**spec)
    say(f"mode-B window {W} case {spec}: q_lens {case.q_lens.tolist()} kv_lens {case.kv_len.tolist()}")
    G = case.num_q_heads // case.num_kv_heads
    meta = bcp.StepMeta(**DeviceCase(case).meta_kwargs())
    assert (bcp.num_q_tiles(meta) == -(-case.max_q_len // (64 // G))) == narrow
    O_ref, L_ref = oracle_attention(case, window=W, q_pos=q_pos, kv_pos=kv_pos)
    out, lse, _ = run(case, q_pos, kv_pos, W)
    assert_close(out, O_ref, case.dtype, lse, L_ref, what=f"mode B window {W}")
    out2, _, _ = run(case, q_pos, kv_pos, W, plan=False)
    assert torch.equal(out.view(torch.uint8) if out.dtype == torch.bfloat16 else out,
                       out2.view(torch.uint8) if out2.dtype == torch.bfloat16 else out2)


@pytest.mark.parametrize("seed,W,tq,tk,shape", [
    (111, 9, 64, 64, dict(prompt=300, canvas=64)), (112, 40, 16, 32, {}), (113, 3, 7, 5, {}),
    (114, 100, 64, 64, dict(prompt=400, canvas=64, n_canvas=4))])
def test_mode_B_window_tile_classes(seed, W, tq, tk, shape):
    case, (q_pos, kv_pos) = canvas_case(seed, G=4, d=64, P=8, **shape)
    dc = DeviceCase(case)
    meta = bcp.StepMeta(**dict(dc.meta_kwargs(), tile_q=tq, tile_k=tk, check=True, window=W))
    nqt, nkt = bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)
    tc = torch.full((case.batch, nqt, nkt), 255, dtype=torch.uint8, device="cuda")
    bcp.build_tile_mask(meta, tile_class=tc)
    torch.cuda.synchronize()
    ref = oracle_tiles(case, tq, tk, window=W, q_pos=q_pos, kv_pos=kv_pos)
    np.testing.assert_array_equal(tc.cpu().numpy(), ref)
    # the window must actually cut something in these cases
    assert (ref != oracle_tiles(case, tq, tk)).any()


def test_C4_multi_canvas_window_sampled():
    # C4's multi-canvas layout with its positions, W = 512: canvases far from the prompt's
    # start lose its early part.
    case = config(4)
    q_pos, kv_pos = case.q_pos, case.kv_pos
    rows = {s: np.unique(np.concatenate([[0, int(case.q_lens[s]) - 1], np.random.default_rng(s).integers(
        0, int(case.q_lens[s]), 10)])) for s in (0, 5, 15)}
    O_ref, L_ref = oracle_attention(case, rows=rows, window=512, q_pos=q_pos, kv_pos=kv_pos)
    out, lse, _ = run(case, q_pos, kv_pos, 512)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C4 window 512 sampled")
    assert torch.isfinite(out.float()).all()


def test_position_tags_commit_with_the_ids():
    case, (q_pos, kv_pos) = canvas_case(121, G=4, d=64, P=8)
    dc = DeviceCase(case)
    qp = torch.from_numpy(q_pos).cuda()
    kp = torch.from_numpy(kv_pos).cuda()
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    kvb = dc.kv_blk.clone()
    bcp.kv_commit_block(meta, dc.k_new, dc.v_new, dc.cu_q, dc.kv_len, dc.k_cache, dc.v_cache, case.total_q,
                        src_blk=dc.q_blk, kv_blk_out=kvb)
    bcp.kv_commit_block(meta, None, None, dc.cu_q, dc.kv_len, dc.k_cache, dc.v_cache, case.total_q,
                        src_blk=qp, kv_blk_out=kp, n_src=case.total_q)
    torch.cuda.synchronize()
    _, _, ref_blk, ref_pos = oracle.commit(case.k_cache, case.v_cache, case.k_new, case.v_new, case.cu_q,
                                           case.kv_len, case.page_table, case.page_size, case.num_pages,
                                           kv_blk=case.kv_blk, src_blk=case.q_blk, kv_pos=kv_pos, src_pos=q_pos)
    np.testing.assert_array_equal(kvb.cpu().numpy(), ref_blk)
    np.testing.assert_array_equal(kp.cpu().numpy(), ref_pos)
