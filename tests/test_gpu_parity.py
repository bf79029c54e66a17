"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact for tile classes, page translation and the commit scatter; within max-abs 1e-2
and mean-abs 1e-3 for bf16 attention outputs and max-abs 1e-4 for float32 inputs. Small
cases span several tiles with ragged tails; the named workloads run at full size, with
every output compared where the oracle is cheap (C1, C2, C4) and sampled rows where it
is not (C3, C5). Every call goes through the C ABI via the Python binding.
"""
import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
import oracle
from tests.oracle_helpers import oracle_attention, oracle_tiles
from workloads import bf16_bits, config, make_case, multi_canvas_structure
from workloads.device import DeviceCase, to_host_bits

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS = 1e-2, 1e-3, 1e-4


def say(*a):
    print(*a, flush=True)


def run_attn(dc, plan=True, check=True, scale=0.0, want_lse=True, stats=None, **meta_over):
    kw = dc.meta_kwargs()
    kw.update(meta_over)
    meta = bcp.StepMeta(**kw, check=check)
    out = torch.full_like(dc.q, float("nan"))
    lse = torch.full(tuple(dc.q.shape[:2]), float("nan"), dtype=torch.float32, device="cuda") if want_lse else None
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    plan_t = None
    if plan:
        plan_t = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
        bcp.build_tile_mask(meta, plan=plan_t)
    bcp.attn_block_causal_paged(meta, dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, out,
                                plan=plan_t, scale=scale, lse=lse, workspace=ws, stats=stats)
    torch.cuda.synchronize()
    return out, lse


def assert_close(out, O_ref, dtype, L=None, L_ref=None, what=""):
    got = out.float().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(O_ref)
    err = np.abs(got[sel] - O_ref[sel])
    assert np.isfinite(got[sel]).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    ratio = mx / max(1e-30, float(np.abs(O_ref[sel]).max()))
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} max-abs/max|O| {ratio:.3e} over {sel.sum()} values")
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    else:
        assert mx <= F32_MAX_ABS, mx
    if L is not None:
        gl = L.cpu().numpy().astype(np.float64)
        s2 = ~np.isnan(L_ref)
        lerr = np.abs(gl[s2] - L_ref[s2]).max()
        say(f"  {what}: lse max-abs {lerr:.3e}")
        assert lerr <= (1e-3 if dtype == "bf16" else 1e-5), lerr


# ------------------------------------------------------------------ small random cases ---

def small_case(seed, dtype="bf16", G=4, Hkv=2, d=128, D=16, P=16, mode="A", batch=3, max_q=70, max_kv=300):
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, max_q + 1, batch)
    q_lens[rng.integers(0, batch)] = max_q           # one sequence at the maximum
    kv_lens = rng.integers(0, max_kv + 1, batch)
    kv_lens[0] = 0                                      # an empty cache
    std = 1.0 / np.sqrt(d)
    if mode == "A":
        return make_case(seed, dtype=dtype, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                         block_size=D, page_size=P, q_lens=q_lens, kv_lens=kv_lens, qkv_std=std, rng=rng)
    qb = [np.sort(rng.integers(1, 5, n)) for n in q_lens]
    kb = [np.sort(rng.integers(0, 5, n)) for n in kv_lens]
    return make_case(seed, dtype=dtype, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                     block_size=1, page_size=P, q_lens=q_lens, kv_lens=kv_lens, q_blk_seqs=qb,
                     kv_blk_seqs=kb, qkv_std=std, rng=rng)


SMALL = [
    dict(seed=1, dtype="bf16", G=4, d=128, D=16, P=16),
    dict(seed=2, dtype="bf16", G=4, d=64, D=64, P=64),
    dict(seed=3, dtype="bf16", G=1, d=128, D=1, P=32),
    dict(seed=4, dtype="bf16", G=2, d=64, D=3, P=16),
    dict(seed=5, dtype="bf16", G=8, d=128, D=256, P=64),
    dict(seed=6, dtype="bf16", G=4, d=128, D=2, P=1),
    dict(seed=7, dtype="bf16", G=4, d=128, D=1, P=16, mode="B"),
    dict(seed=8, dtype="bf16", G=2, d=64, D=1, P=32, mode="B"),
    dict(seed=9, dtype="f32", G=4, d=128, D=16, P=16),
    dict(seed=10, dtype="f32", G=2, d=64, D=5, P=8),
    dict(seed=11, dtype="f32", G=4, d=64, D=1, P=16, mode="B"),
    dict(seed=12, dtype="bf16", G=16, d=128, D=64, P=16, max_q=40, max_kv=2000),
    dict(seed=13, dtype="bf16", G=4, d=128, D=64, P=64, batch=5, max_q=300, max_kv=700),
    dict(seed=14, dtype="bf16", G=4, d=64, D=1, P=12, mode="B"),
    dict(seed=15, dtype="bf16", G=8, d=128, D=1, P=3, mode="B", max_kv=500),
    dict(seed=16, dtype="bf16", G=4, d=128, D=1, P=8, mode="B", max_q=200, max_kv=900),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_attention_small(spec):
    case = small_case(**spec)
    say(f"small case {spec}: q_lens {case.q_lens.tolist()} kv_lens {case.kv_len.tolist()}")
    O_ref, L_ref = oracle_attention(case)
    dc = DeviceCase(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, case.dtype, lse, L_ref, what="plan")
    out2, _ = run_attn(dc, plan=False, want_lse=False)
    assert torch.equal(out.view(torch.uint8) if out.dtype == torch.bfloat16 else out,
                       out2.view(torch.uint8) if out2.dtype == torch.bfloat16 else out2)


def test_attention_poisoned_tails_and_pages():
    """Slots past kv_len in the last page and every unmapped page hold NaN: never read."""
    case = small_case(21, dtype="bf16", G=4, d=128, D=16, P=16)
    for s in range(case.batch):
        n = int(case.kv_len[s])
        pages_used = -(-n // 16)
        for j in range(n, pages_used * 16):
            pg = case.page_table[s, j // 16]
            case.k_cache[pg, j % 16] = 0x7FC0
            case.v_cache[pg, j % 16] = 0x7FC0
    O_ref, _ = oracle_attention(case)
    out, _ = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", what="poisoned")


def test_attention_large_scores():
    """Scores with a large spread (Q and K ~ N(0,4), scale 1/4): the running max grows
    across tiles and the rescale path runs. V keeps the decode workloads' magnitude
    (N(0,1)/sqrt(d)) so the absolute tolerance applies to outputs of the same size."""
    rng = np.random.default_rng(22)
    case = make_case(22, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=32,
                     page_size=16, q_lens=[96, 64], kv_lens=[300, 129], qkv_std=2.0, rng=rng)
    for name in ("v_new", "v_cache"):        # divide V by 16: exact in bf16, NaN stays NaN
        x = (getattr(case, name).astype(np.uint32) << 16).view(np.float32) / np.float32(16.0)
        setattr(case, name, bf16_bits(x))
    O_ref, L_ref = oracle_attention(case, scale=0.25)
    out, lse = run_attn(DeviceCase(case), scale=0.25)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="large-scores")


def test_page_permutation_is_bit_identical():
    """Relabelling physical pages changes nothing, bit for bit: the reduction order depends
    only on the logical order of the keys."""
    case = small_case(23, dtype="bf16", G=4, d=128, D=64, P=16, max_kv=900)
    dc = DeviceCase(case)
    out1, lse1 = run_attn(dc)
    perm = torch.from_numpy(np.random.default_rng(24).permutation(case.num_pages)).cuda()
    inv = torch.argsort(perm)
    dc.k_cache, dc.v_cache = dc.k_cache[inv].contiguous(), dc.v_cache[inv].contiguous()
    pt = dc.page_table.long()
    dc.page_table = torch.where(pt >= 0, perm[pt.clamp(min=0)], pt).int().contiguous()
    out2, lse2 = run_attn(dc)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_prefill_equals_commit_then_decode():
    """Prefill of blocks 0..4 equals committing blocks 0..3 through kv_commit_block and then
    decoding block 4 against the cache (within tolerance; the order of sums differs)."""
    D, P, n = 64, 16, 5 * 64
    rng = np.random.default_rng(25)
    case = make_case(25, dtype="bf16", num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=D,
                     page_size=P, q_lens=[n], kv_lens=[0], qkv_std=1 / np.sqrt(128), rng=rng)
    dc = DeviceCase(case)
    out_pre, _ = run_attn(dc)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    cu_src = torch.tensor([0, 4 * D], dtype=torch.int32, device="cuda")
    dst = torch.zeros(1, dtype=torch.int32, device="cuda")
    bcp.kv_commit_block(meta, dc.k_new, dc.v_new, cu_src, dst, dc.k_cache, dc.v_cache, 4 * D)
    dec = make_case(25, dtype="bf16", num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=D,
                    page_size=P, q_lens=[D], kv_lens=[4 * D], num_pages=case.num_pages, rng=rng)
    dd = DeviceCase(dec)
    dd.q, dd.k_new, dd.v_new = dc.q[4 * D:].contiguous(), dc.k_new[4 * D:].contiguous(), dc.v_new[4 * D:].contiguous()
    dd.k_cache, dd.v_cache, dd.page_table = dc.k_cache, dc.v_cache, dc.page_table
    out_dec, _ = run_attn(dd)
    err = (out_dec.float() - out_pre[4 * D:].float()).abs()
    say(f"  prefill vs commit+decode: max {err.max().item():.3e} mean {err.mean().item():.3e}")
    assert err.max().item() <= BF16_MAX_ABS and err.mean().item() <= BF16_MEAN_ABS


# ------------------------------------------------------------------ named workloads ------

@pytest.fixture(scope="module")
def workloads():
    cache = {}

    def get(n):
        if n not in cache:
            say(f"generating workload C{n}")
            cache[n] = config(n)
        return cache[n]
    return get


def test_C1_tiny_fp32(workloads):
    case = workloads(1)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "f32", lse, L_ref, what="C1")


def test_C2_decode_full(workloads):
    case = workloads(2)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C2")


def test_C4_multi_canvas_full(workloads):
    case = workloads(4)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C4")


def test_C5_long_context_sampled(workloads):
    case = workloads(5)
    order = np.argsort(case.kv_len)
    seqs = list(order[:4]) + list(order[-4:]) + list(order[28:32])
    rows = {int(s): np.array([0, 17, 38, 63]) for s in seqs}
    O_ref, L_ref = oracle_attention(case, rows=rows)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C5 sampled")
    assert torch.isfinite(out.float()).all()


def test_C3_prefill_sampled(workloads):
    case = workloads(3)
    rng = np.random.default_rng(3003)
    rows = {s: np.unique(np.concatenate([[0, 63, 64, 8191], rng.integers(0, 8192, 28)])) for s in range(4)}
    O_ref, L_ref = oracle_attention(case, rows=rows)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C3 sampled")
    assert torch.isfinite(out.float()).all()


def test_items_longer_than_one_window():
    # 4 sequences x 65 q-tiles, each over 16384 committed keys and a 4160-row prompt, one kv
    # head: more than 256 (unit, head) pairs and more than 65536 visits, so the stream-K
    # ranges hold over 256 tiles and some items span two metadata windows of the kernel.
    rng = np.random.default_rng(4242)
    case = make_case(4242, dtype="bf16", num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=64,
                     page_size=64, q_lens=[4160] * 4, kv_lens=[16384] * 4, qkv_std=1 / 8, rng=rng)
    dc = DeviceCase(case)
    w, nqt, nkt = _plan_words(case, dc)
    U = case.batch * nqt
    items_off = 8 + U + U * nkt + U + 1 + N_WGS + 1
    items = w[items_off:items_off + ITEM_WORDS * int(w[0])].reshape(-1, ITEM_WORDS)
    assert (items[:, 3] - items[:, 2]).max() > 256
    rows = {s: np.unique(np.concatenate([[0, 63, 64, 4159], rng.integers(0, 4160, 12)])) for s in range(4)}
    O_ref, L_ref = oracle_attention(case, rows=rows)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="two-window items")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sequences_without_live_rows(dtype):
    # Sequences with no live rows (and one with neither live rows nor cache) among others:
    # they own no q-tile work and must not disturb the rest.
    rng = np.random.default_rng(77)
    case = make_case(77, dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                     page_size=16, q_lens=[0, 37, 0, 64, 0], kv_lens=[100, 250, 0, 0, 300],
                     qkv_std=1 / np.sqrt(128), rng=rng)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, dtype, lse, L_ref, what="empty sequences")


# ------------------------------------------------------------------ tile classes ---------

def tile_case_list():
    return [
        ("fig-blockmask", dict(tokens=6, D=2), 2, 2),
        ("fig-prefill", dict(tokens=16, D=4), 4, 4),
        ("unaligned", dict(tokens=16, D=4), 4, 8),
    ]


@pytest.mark.parametrize("name,spec,tq,tk", tile_case_list(), ids=[c[0] for c in tile_case_list()])
def test_tile_classes_page_figures(name, spec, tq, tk):
    case = make_case(1, dtype="bf16", num_q_heads=1, num_kv_heads=1, head_dim=64, block_size=spec["D"],
                     page_size=4, q_lens=[spec["tokens"]], kv_lens=[0])
    check_tiles(case, tq, tk)


def check_tiles(case, tq, tk, with_plan=False, window=0):
    # With a plan requested too, the classes and pages must be the same.
    dc = DeviceCase(case)
    meta = bcp.StepMeta(**dc.meta_kwargs(), tile_q=tq, tile_k=tk, check=True, window=window)
    nqt, nkt = bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)
    nct = -(-case.max_kv_len // tk)
    ppt = max(1, tk // case.page_size)
    tc = torch.full((case.batch, nqt, nkt), 255, dtype=torch.uint8, device="cuda")
    pp = torch.full((case.batch, nct, ppt), -7, dtype=torch.int32, device="cuda") if nct else None
    plan_t = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda") if with_plan else None
    bcp.build_tile_mask(meta, tile_class=tc, phys_page=pp, plan=plan_t)
    torch.cuda.synchronize()
    ref = oracle_tiles(case, tq, tk, window=window or None)
    got = tc.cpu().numpy()
    assert got.shape == ref.shape
    np.testing.assert_array_equal(got, ref)
    if nct:
        np.testing.assert_array_equal(pp.cpu().numpy(), oracle.phys_page(case.page_table, case.kv_len,
                                                                          case.page_size, tk, nct))
    return got


@pytest.mark.parametrize("seed,mode,tq,tk,P", [(31, "A", 64, 64, 16), (32, "B", 64, 64, 16),
                                                (33, "A", 16, 32, 8), (34, "B", 32, 16, 32),
                                                (35, "A", 128, 64, 64), (36, "B", 7, 5, 3)])
def test_tile_classes_random(seed, mode, tq, tk, P):
    case = small_case(seed, G=4, d=64, D=5, P=P, mode=mode, max_q=150, max_kv=400)
    check_tiles(case, tq, tk)
    if (tq, tk) == (64, 64):
        check_tiles(case, tq, tk, with_plan=True)


@pytest.mark.parametrize("n", [1, 2, 4, 5, 3])
def test_tile_classes_workloads(workloads, n):
    case = workloads(n)
    G = case.num_q_heads // case.num_kv_heads
    check_tiles(case, 256 // G, 64, with_plan=True)
    got = check_tiles(case, 64, 64)
    if n == 3:
        assert (got == bcp.BCP_TILE_FULL).sum() == 4 * 8256 and (got == bcp.BCP_TILE_PARTIAL).sum() == 0


# ------------------------------------------------------------------ sliding window -------
# Mode A with a band of W positions (committed row j at position j, live row i at
# kv_len + i): tiles wholly outside the band are SKIP, tiles it cuts are PARTIAL.

WINDOW_TILES = [(41, 64, 64, 16, 1), (42, 64, 64, 16, 37), (43, 16, 32, 8, 64), (44, 128, 64, 64, 200),
                (45, 7, 5, 3, 9), (46, 64, 64, 16, 100000)]


@pytest.mark.parametrize("seed,tq,tk,P,W", WINDOW_TILES)
def test_window_tile_classes(seed, tq, tk, P, W):
    case = small_case(seed, G=4, d=64, D=5, P=P, max_q=150, max_kv=400)
    got = check_tiles(case, tq, tk, window=W)
    if (tq, tk) == (64, 64):
        check_tiles(case, tq, tk, with_plan=True, window=W)
    if W == 100000:   # a band wider than any sequence changes no class
        np.testing.assert_array_equal(got, oracle_tiles(case, tq, tk))


WINDOW_SMALL = [
    dict(seed=51, dtype="bf16", G=4, d=128, D=16, P=16, W=1),
    dict(seed=52, dtype="bf16", G=4, d=128, D=16, P=16, W=23),
    dict(seed=53, dtype="bf16", G=2, d=64, D=3, P=16, W=64),
    dict(seed=54, dtype="bf16", G=8, d=128, D=64, P=64, W=130),
    dict(seed=55, dtype="bf16", G=4, d=64, D=1, P=8, W=5),
    dict(seed=56, dtype="bf16", G=4, d=128, D=64, P=64, W=257, batch=5, max_q=300, max_kv=700),
    dict(seed=57, dtype="f32", G=4, d=128, D=16, P=16, W=40),
    dict(seed=58, dtype="f32", G=2, d=64, D=5, P=8, W=3),
]


@pytest.mark.parametrize("spec", WINDOW_SMALL, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_window_attention_small(spec):
    spec = dict(spec)
    W = spec.pop("W")
    case = small_case(**spec)
    say(f"window {W} case {spec}: q_lens {case.q_lens.tolist()} kv_lens {case.kv_len.tolist()}")
    O_ref, L_ref = oracle_attention(case, window=W)
    dc = DeviceCase(case)
    out, lse = run_attn(dc, window=W)
    assert_close(out, O_ref, case.dtype, lse, L_ref, what=f"window {W}")
    out2, _ = run_attn(dc, plan=False, want_lse=False, window=W)
    assert torch.equal(out.view(torch.uint8) if out.dtype == torch.bfloat16 else out,
                       out2.view(torch.uint8) if out2.dtype == torch.bfloat16 else out2)


def test_window_wider_than_every_sequence_is_bit_identical():
    case = small_case(59, G=4, d=128, D=16, P=16, batch=4, max_q=130, max_kv=500)
    dc = DeviceCase(case)
    out, lse = run_attn(dc)
    outw, lsew = run_attn(dc, window=int(case.kv_len.max()) + case.max_q_len)
    assert torch.equal(out.view(torch.uint8), outw.view(torch.uint8))
    assert torch.equal(lse, lsew)


def test_window_C2_decode_full(workloads):
    case = workloads(2)
    O_ref, L_ref = oracle_attention(case, window=1024)
    out, lse = run_attn(DeviceCase(case), window=1024)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C2 window 1024")


def test_window_C5_long_context_sampled(workloads):
    case = workloads(5)
    order = np.argsort(case.kv_len)
    seqs = list(order[:4]) + list(order[-4:]) + list(order[28:32])
    rows = {int(s): np.array([0, 17, 38, 63]) for s in seqs}
    O_ref, L_ref = oracle_attention(case, rows=rows, window=4096)
    out, lse = run_attn(DeviceCase(case), window=4096)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C5 window 4096 sampled")
    assert torch.isfinite(out.float()).all()


# Step-plan invariants. The plan is the library's internal work list (layout documented in
# its internal header, mirrored here): the (kv head, unit, key tile) visits are cut into
# contiguous ranges of near-equal length, one per workgroup; every pair's tiles are covered
# exactly once, in order; pieces of a cut pair own distinct partial slots.
N_WGS, ITEM_WORDS, MAX_SLOTS, ITEM_COST = 256, 8, 512, 5


def _plan_words(case, dc):
    meta = bcp.StepMeta(**dc.meta_kwargs())
    plan_t = torch.zeros(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    bcp.build_tile_mask(meta, plan=plan_t)
    torch.cuda.synchronize()
    return plan_t.view(torch.int32).cpu().numpy(), bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)


@pytest.mark.parametrize("n", [1, 2, 4, 5, 3])
def test_plan_ranges_cover_every_visit_once(workloads, n):
    case = workloads(n)
    w, nqt, nkt = _plan_words(case, DeviceCase(case))
    U, hkv = case.batch * nqt, case.num_kv_heads
    cnt_off = 8
    list_off = cnt_off + U
    upre_off = list_off + U * nkt
    wg_off = upre_off + U + 1
    items_off = wg_off + N_WGS + 1
    max_items = U * hkv + N_WGS
    split_off = items_off + ITEM_WORDS * max_items
    n_items, n_split, n_wg, total = int(w[0]), int(w[1]), int(w[2]), int(w[3])
    cnt = w[cnt_off:cnt_off + U].astype(np.int64)
    assert total == cnt.sum()
    # The tile counts agree with the oracle's classes (non-skipped tiles per unit).
    cls = oracle_tiles(case, 256 // (case.num_q_heads // hkv), 64)
    np.testing.assert_array_equal(cnt, (cls != 0).reshape(U, -1).sum(axis=1))
    wg = w[wg_off:wg_off + N_WGS + 1]
    assert wg[0] == 0 and wg[-1] == n_items and np.all(np.diff(wg) >= 0)
    items = w[items_off:items_off + ITEM_WORDS * n_items].reshape(n_items, ITEM_WORDS)
    covered = {}
    loads = np.zeros(N_WGS, dtype=np.int64)
    slots = []
    for k in range(N_WGS):
        for it in items[wg[k]:wg[k + 1]]:
            u, g, ob, oe, ps = (int(x) for x in it[:5])
            assert 0 <= u < U and 0 <= g < hkv and 0 <= ob < oe <= cnt[u]
            covered.setdefault((u, g), []).append((ob, oe, ps))
            loads[k] += oe - ob
            if ps >= 0:
                slots.append(ps)
    for u in range(U):
        for g in range(hkv):
            pieces = covered.get((u, g), [])
            if cnt[u] == 0:
                assert not pieces
                continue
            assert pieces[0][0] == 0 and pieces[-1][1] == cnt[u]
            assert all(a[1] == b[0] for a, b in zip(pieces, pieces[1:]))
            assert (len(pieces) == 1) == (pieces[0][2] < 0)
    assert len(slots) == len(set(slots)) and (not slots or max(slots) < MAX_SLOTS)
    # Each item carries its sequence's live rows and committed length (clamped to the pages).
    for it in items:
        s = int(it[0]) // nqt
        kv_cap = case.max_pages_per_seq * case.page_size
        assert list(it[5:8]) == [case.cu_q[s], case.cu_q[s + 1] - case.cu_q[s], min(case.kv_len[s], kv_cap)]
    # Range records: item bounds, and a copy of the first item of every non-empty range.
    rng_off = split_off + 4 * N_WGS
    rec = w[rng_off:rng_off + 12 * N_WGS].reshape(N_WGS, 12)
    np.testing.assert_array_equal(rec[:, 0], wg[:-1])
    np.testing.assert_array_equal(rec[:, 1], wg[1:])
    for k in range(N_WGS):
        if wg[k] < wg[k + 1]:
            np.testing.assert_array_equal(rec[k, 2:10], items[wg[k]])
    splits = w[split_off:split_off + 4 * n_split].reshape(n_split, 4)
    for u, g, ps0, npieces in splits:
        assert [p[2] for p in covered[(int(u), int(g))]] == list(range(ps0, ps0 + npieces))
    used = loads[:n_wg]
    assert loads[n_wg:].sum() == 0 and used.sum() == total * hkv
    if U * hkv > N_WGS:
        # Many pairs: the visits, each pair preceded by ITEM_COST start-up positions, are cut
        # into ranges that differ by at most one position. Counting ITEM_COST for each pair
        # that starts in a range is off by at most ITEM_COST at either end.
        starts = np.zeros(N_WGS, dtype=np.int64)
        for k in range(N_WGS):
            starts[k] = sum(1 for it in items[wg[k]:wg[k + 1]] if it[2] == 0)
        cost = (loads + ITEM_COST * starts)[:n_wg]
        assert cost.max() - cost.min() <= 2 * ITEM_COST + 1
    else:
        # Few pairs: each is cut into near-equal chunks, one per range.
        assert n_wg == n_items and used.max() <= 1.5 * used.mean() + 1


def test_stats_count_tiles(workloads):
    case = workloads(4)
    dc = DeviceCase(case)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    run_attn(dc, stats=stats)
    s = stats.cpu().numpy()
    ref = oracle_tiles(case, 64, 64)
    H = case.num_kv_heads
    assert s[0] == H * (ref == 2).sum() and s[1] == H * (ref == 1).sum() and s[2] == H * (ref == 0).sum()


# ------------------------------------------------------------------ commit ---------------

def commit_and_compare(case, cu_src, dst_start, src_row=None, src_blk=None, with_blk=False):
    dc = DeviceCase(case)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    total = int(cu_src[-1])
    kvb0 = case.kv_blk if case.kv_blk is not None else np.full(case.num_pages * case.page_size, -1, np.int32)
    kvb = torch.from_numpy(kvb0.copy()).cuda() if with_blk else None
    t = lambda x: None if x is None else torch.from_numpy(np.asarray(x, np.int32)).cuda()
    bcp.kv_commit_block(meta, dc.k_new, dc.v_new, t(cu_src), t(dst_start), dc.k_cache, dc.v_cache, total,
                        src_row=t(src_row), src_blk=t(src_blk) if with_blk else None, kv_blk_out=kvb)
    torch.cuda.synchronize()
    kc, vc, kb = oracle.commit(case.k_cache, case.v_cache, case.k_new, case.v_new, cu_src, dst_start,
                               case.page_table, case.page_size, case.num_pages, src_row=src_row,
                               kv_blk=kvb0 if with_blk else None, src_blk=src_blk if with_blk else None)
    gk, gv = to_host_bits(dc.k_cache), to_host_bits(dc.v_cache)
    if case.dtype == "f32":
        gk, gv, kc, vc = gk.view(np.uint32), gv.view(np.uint32), kc.view(np.uint32), vc.view(np.uint32)
    np.testing.assert_array_equal(gk, kc)
    np.testing.assert_array_equal(gv, vc)
    if with_blk:
        np.testing.assert_array_equal(kvb.cpu().numpy(), kb)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_commit_small(dtype):
    case = small_case(41, dtype=dtype, G=2, d=64, D=4, P=8)
    rng = np.random.default_rng(42)
    n = case.q_lens
    take = np.array([rng.integers(0, k + 1) for k in n])        # commit a prefix of each sequence
    cu_src = np.concatenate([[0], np.cumsum(take)]).astype(np.int32)
    src_row = np.concatenate([case.cu_q[s] + rng.permutation(n[s])[:take[s]] for s in range(case.batch)]).astype(np.int32)
    src_blk = rng.integers(0, 9, case.total_q).astype(np.int32)
    commit_and_compare(case, cu_src, case.kv_len, src_row=src_row, src_blk=src_blk, with_blk=True)


def test_commit_C2_block(workloads):
    case = workloads(2)
    commit_and_compare(case, case.cu_q, case.kv_len)


def test_commit_C3_all_blocks(workloads):
    case = workloads(3)
    commit_and_compare(case, case.cu_q, np.zeros(4, np.int32))


# ------------------------------------------------------------------ checked mode ---------

def test_checked_mode_rejects_bad_metadata():
    case = small_case(51, G=4, d=64, D=8, P=8)
    dc = DeviceCase(case)
    s = int(np.argmax(case.kv_len))
    pt = dc.page_table.clone()
    pt[s, 0] = case.num_pages                     # a page past the pool
    with pytest.raises(bcp.BcpError) as e:
        run_attn(dc, page_table=pt)
    assert e.value.code == bcp.BCP_E_RANGE
    kvl = dc.kv_len.clone()
    kvl[0] = case.max_kv_len + 1
    with pytest.raises(bcp.BcpError) as e:
        run_attn(dc, kv_len=kvl)
    assert e.value.code == bcp.BCP_E_RANGE
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    cu = torch.tensor([0, 1, 2] + [2] * (case.batch - 2), dtype=torch.int32, device="cuda")
    dst = torch.zeros(case.batch, dtype=torch.int32, device="cuda")
    row = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    pt2 = dc.page_table.clone()
    pt2[1, 0] = pt2[0, 0]                          # two sequences share a destination page
    meta2 = bcp.StepMeta(**{**dc.meta_kwargs(), "page_table": pt2}, check=True)
    with pytest.raises(bcp.BcpError) as e:
        bcp.kv_commit_block(meta2, dc.k_new, dc.v_new, cu, dst, dc.k_cache, dc.v_cache, 2, src_row=row)
    assert e.value.code == bcp.BCP_E_RANGE
    del meta
