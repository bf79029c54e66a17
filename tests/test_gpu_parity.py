"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact for tile classes, page translation and the commit scatter; within max-abs 1e-2
and mean-abs 1e-3 for bf16 attention outputs and max-abs 1e-4 for float32 inputs. Those
absolute bounds are loose where the outputs are small (the decode workloads' outputs are
of order 1e-2), so every comparison also bounds the error relative to the output's own
scale: max-abs / max|O| and mean-abs / mean|O| within 1e-2 for bf16 (1e-4 for float32).
bf16 rounding of the output alone is 2^-9 relative at most, so this costs nothing when
the kernel is right, while a dropped key tile or a mis-masked block edge fails it. Small
cases span several tiles with ragged tails; the named workloads run at full size, with
every output compared where the oracle is cheap (C1, C2, C4, C5 on eight rows of every
sequence) and sampled rows where it is not (C3). Every call goes through the C ABI via
the Python binding.
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
BF16_REL, F32_REL = 1e-2, 1e-4      # max-abs / max|O| and mean-abs / mean|O|


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


def assert_close(out, O_ref, dtype, L=None, L_ref=None, what="", abs_gate=True):
    """abs_gate=False keeps only the scale-free bounds: for stress inputs whose values are
    far larger than the workloads' (the absolute bounds are stated for those)."""
    got = out.float().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(O_ref)
    err = np.abs(got[sel] - O_ref[sel])
    assert np.isfinite(got[sel]).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    ref_abs = np.abs(O_ref[sel])
    ratio = mx / max(1e-300, float(ref_abs.max()))
    mratio = mean / max(1e-300, float(ref_abs.mean()))
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} max-abs/max|O| {ratio:.3e} "
        f"mean-abs/mean|O| {mratio:.3e} over {sel.sum()} values")
    rel = BF16_REL if dtype == "bf16" else F32_REL
    assert ratio <= rel and mratio <= rel, (ratio, mratio)
    if abs_gate and dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (mx, mean)
    elif abs_gate:
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
    # Mode B: block ids sorted in row order ("B"), or in promotion order ("Bu": ids in no
    # order, as when entries are promoted one step late and the arena is compacted).
    qb = [rng.integers(1, 5, n) for n in q_lens]
    kb = [rng.integers(0, 5, n) for n in kv_lens]
    if mode == "B":
        qb, kb = [np.sort(b) for b in qb], [np.sort(b) for b in kb]
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
    # promotion order: block ids of live and committed rows in no particular order
    dict(seed=17, dtype="bf16", G=4, d=128, D=1, P=16, mode="Bu", max_q=200, max_kv=900),
    dict(seed=18, dtype="bf16", G=8, d=64, D=1, P=3, mode="Bu", max_kv=500),
    dict(seed=19, dtype="bf16", G=2, d=128, D=1, P=64, mode="Bu", batch=4, max_q=300, max_kv=1500),
    dict(seed=20, dtype="f32", G=4, d=64, D=1, P=8, mode="Bu"),
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


def bf16_float(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def sorted_score_case(seed, q_lens, kv_lens, D=32, P=16, Hq=8, Hkv=2, d=64, common=32.0):
    """Large scores whose row maximum grows across the key tiles: Q and K ~ N(0,4), every
    query shares a strong component along one direction u, and each sequence's keys (with
    their values, per kv head) are sorted along u in logical order -- cached rows in page
    order, then the live rows -- so the scores rise from key to key by tens of log2 units
    and the online softmax rescales again and again."""
    rng = np.random.default_rng(seed)
    case = make_case(seed, dtype="bf16", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, block_size=D,
                     page_size=P, q_lens=q_lens, kv_lens=kv_lens, qkv_std=2.0, rng=rng)
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    case.q = bf16_bits(bf16_float(case.q) + np.float32(common) * u)
    for s in range(case.batch):
        n = int(case.kv_len[s])
        j = np.arange(n)
        pg, sl = case.page_table[s, j // P], j % P
        K, V = bf16_float(case.k_cache[pg, sl]), bf16_float(case.v_cache[pg, sl])
        lo, hi = int(case.cu_q[s]), int(case.cu_q[s + 1])
        Kn, Vn = bf16_float(case.k_new[lo:hi]), bf16_float(case.v_new[lo:hi])
        for h in range(Hkv):
            o = np.argsort(K[:, h] @ u, kind="stable")
            K[:, h], V[:, h] = K[o, h], V[o, h]
            o = np.argsort(Kn[:, h] @ u, kind="stable")
            Kn[:, h], Vn[:, h] = Kn[o, h], Vn[o, h]
        case.k_cache[pg, sl], case.v_cache[pg, sl] = bf16_bits(K), bf16_bits(V)
        case.k_new[lo:hi], case.v_new[lo:hi] = bf16_bits(Kn), bf16_bits(Vn)
    return case


def test_attention_large_scores():
    """Scores spanning about +-45 log2 units that grow along the key order (sorted keys), so
    the running max moves by more than the lazy threshold many times per row. The values
    are N(0,4) as drawn, so outputs reach several units: the gate is the scale-free one
    (the workloads' absolute bounds are stated for their own value scale) plus the LSE."""
    case = sorted_score_case(22, q_lens=[96, 64], kv_lens=[300, 129])
    O_ref, L_ref = oracle_attention(case, scale=0.25)
    out, lse = run_attn(DeviceCase(case), scale=0.25)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="large-scores", abs_gate=False)


def offset_score_case(seed, offsets, q_lens, kv_lens, G=4, Hkv=2, d=128, D=64, P=16):
    """Scores shifted far from zero: every key (cached and live) carries a component c*u
    along one unit direction u, and query head h a component a_h*u, so each score of head h
    is offset by about offsets[h % len(offsets)] log2 units (after the 1/sqrt(d) scale) on
    top of a spread of a few units. Far below zero the exponentials underflow against a
    reference near 0; far above, they overflow: the online softmax has to move its
    reference before it can use a tile."""
    rng = np.random.default_rng(seed)
    case = make_case(seed, dtype="bf16", num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d, block_size=D,
                     page_size=P, q_lens=q_lens, kv_lens=kv_lens, qkv_std=1 / np.sqrt(d), rng=rng)
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    c = np.float32(48.0)
    sl2 = np.log2(np.e) / np.sqrt(d)
    a = np.array([offsets[h % len(offsets)] / (sl2 * c) for h in range(G * Hkv)], dtype=np.float32)
    case.q = bf16_bits(bf16_float(case.q) + a[None, :, None] * u)
    case.k_new = bf16_bits(bf16_float(case.k_new) + c * u)
    used = np.zeros(case.k_cache.shape[:2], dtype=bool)     # only mapped, committed slots
    for s in range(case.batch):
        j = np.arange(int(case.kv_len[s]))
        used[case.page_table[s, j // P], j % P] = True
    kc = bf16_float(case.k_cache)
    kc[used] += c * u
    case.k_cache = np.where(used[..., None, None], bf16_bits(np.nan_to_num(kc)), case.k_cache)
    return case


@pytest.mark.parametrize("offsets", [(-300.0,), (-100.0,), (300.0,), (-300.0, 300.0, 0.0, -90.0)],
                         ids=["minus300", "minus100", "plus300", "mixed"])
@pytest.mark.parametrize("narrow", [False, True], ids=["wide", "narrow"])
def test_scores_far_from_zero(offsets, narrow):
    """Rows whose scores all sit hundreds of log2 units below or above zero (and, mixed,
    heads of either kind in one wave) match the oracle, which subtracts each row's true max.
    Wide q-tiles (64 live rows per sequence) and narrow ones (at most 16 positions)."""
    q_lens, kv_lens = ([64, 64, 40], [700, 129, 0]) if not narrow else ([9, 5, 16], [700, 129, 0])
    case = offset_score_case(31 + len(offsets), offsets, q_lens, kv_lens)
    dc = DeviceCase(case)
    assert (bcp.num_q_tiles(bcp.StepMeta(**dc.meta_kwargs())) == 1) and (case.max_q_len * 4 <= 64) == narrow
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, "bf16", lse, L_ref, what=f"scores offset {offsets}")


def test_large_scores_grow_across_tiles():
    """The stress case really moves the row max across tiles: for most query rows the max
    over each successive 64-key tile of the cached keys rises, and overall by > 8 log2 units."""
    case = sorted_score_case(22, q_lens=[96, 64], kv_lens=[300, 129])
    s, P = 0, case.page_size
    n = int(case.kv_len[s])
    j = np.arange(n)
    K = bf16_float(case.k_cache[case.page_table[s, j // P], j % P]).astype(np.float64)   # [n, Hkv, d]
    Q = bf16_float(case.q[:int(case.cu_q[1])]).astype(np.float64)
    S = 0.25 * np.log2(np.e) * np.einsum("qd,kd->qk", Q[:, 0], K[:, 0])    # head 0, kv head 0
    tmax = np.stack([S[:, t:t + 64].max(axis=1) for t in range(0, n, 64)], axis=1)
    runmax = np.maximum.accumulate(tmax, axis=1)
    grows = (np.diff(runmax, axis=1) > 8).sum(axis=1)
    assert np.median(grows) >= 2, grows


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


def test_C2_shape_unit_normal_full():
    """C2's shape (8 sequences, 32/8 heads, d 128, D 64, committed 64 * U{8..64}, pages of 64
    over a 4096-page pool) with Q/K/V ~ N(0,1) instead of N(0,1)/sqrt(128). The outputs are
    about 50 times larger than C2's (max|O| 0.45 against 0.008), so the absolute bounds
    (max-abs 1e-2, mean-abs 1e-3) are a few percent of the output's scale instead of more
    than all of it. (Much larger outputs cannot meet them at all: one bf16 rounding step is
    already 0.0156 at |O| = 4.)"""
    rng = np.random.default_rng(2002)
    kv = 64 * rng.integers(8, 65, size=8)
    case = make_case(2002, dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=64,
                     page_size=64, q_lens=[64] * 8, kv_lens=kv, num_pages=4096, qkv_std=1.0, rng=rng)
    O_ref, L_ref = oracle_attention(case)
    say(f"  C2 shape, N(0,1): max|O| {np.abs(O_ref).max():.3f} mean|O| {np.abs(O_ref).mean():.3f}")
    assert np.abs(O_ref).max() > 0.2
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C2 shape N(0,1)")


def test_C4_multi_canvas_full(workloads):
    case = workloads(4)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C4")


def test_C5_long_context_every_sequence(workloads):
    """All 64 sequences, eight rows each: both ends of the block, and six drawn rows."""
    case = workloads(5)
    rng = np.random.default_rng(5005)
    rows = {s: np.unique(np.concatenate([[0, 63], rng.choice(np.arange(1, 63), 6, replace=False)]))
            for s in range(case.batch)}
    O_ref, L_ref = oracle_attention(case, rows=rows)
    out, lse = run_attn(DeviceCase(case))
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C5, 8 rows of every sequence")
    assert torch.isfinite(out.float()).all()


def test_C3_prefill_sampled(workloads):
    """The first and last row of every one of the 128 blocks of every sequence (each block
    edge of the mask, from both sides) and 32 drawn rows per sequence."""
    case = workloads(3)
    rng = np.random.default_rng(3003)
    rows = {s: np.unique(np.concatenate([np.arange(0, 8192, 64), np.arange(63, 8192, 64), rng.integers(0, 8192, 32)]))
            for s in range(4)}
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
    items_off = HDR_WORDS + 12 * N_WGS + 4 * N_WGS + U + U * nkt + U + 1 + N_WGS + 1
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
                                                (35, "A", 128, 64, 64), (36, "B", 7, 5, 3),
                                                (37, "Bu", 64, 64, 16), (38, "Bu", 16, 32, 8)])
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
N_WGS, ITEM_WORDS, MAX_SLOTS, ITEM_COST, HDR_WORDS = 256, 8, 512, 5, 16


def _plan_words(case, dc):
    meta = bcp.StepMeta(**dc.meta_kwargs())
    plan_t = torch.zeros(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    bcp.build_tile_mask(meta, plan=plan_t)
    torch.cuda.synchronize()
    return plan_t.view(torch.int32).cpu().numpy(), bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)


@pytest.mark.parametrize("vexp", [26, -100], ids=["values_2e26", "values_2e-100"])
@pytest.mark.parametrize("q_lens", [[64, 64], [9, 5]], ids=["wide", "narrow"])
@pytest.mark.parametrize("d", [128, 64])
def test_split_partials_keep_the_value_scale(vexp, q_lens, d):
    """Split pieces store their partial rows in 16 bits, each row scaled by a power of two into
    range: outputs reaching 5e5 (past fp16's largest value) and of order 1e-32 (far below its
    smallest) come back at their scale. The step is cut into split pieces (checked in the
    plan header), and the result is compared scale-free with the oracle."""
    rng = np.random.default_rng(40 + abs(vexp))
    case = make_case(40, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=d, block_size=64,
                     page_size=16, q_lens=q_lens, kv_lens=[1500, 900], qkv_std=1 / np.sqrt(d), rng=rng)
    f = np.float32(2.0 ** vexp)
    case.v_new = bf16_bits(bf16_float(case.v_new) * f)
    case.v_cache = bf16_bits(bf16_float(case.v_cache) * f)   # NaN slots stay NaN
    dc = DeviceCase(case)
    w, _, _ = _plan_words(case, dc)
    assert w[1] > 0, "the step has no split pieces"
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, "bf16", lse, L_ref, what=f"values x 2^{vexp}", abs_gate=False)


@pytest.mark.parametrize("n", [1, 2, 4, 5, 3])
def test_plan_ranges_cover_every_visit_once(workloads, n):
    case = workloads(n)
    w, nqt, nkt = _plan_words(case, DeviceCase(case))
    U, hkv = case.batch * nqt, case.num_kv_heads
    rng_off = HDR_WORDS
    split_off = rng_off + 12 * N_WGS
    cnt_off = split_off + 4 * N_WGS
    list_off = cnt_off + U
    upre_off = list_off + U * nkt
    wg_off = upre_off + U + 1
    items_off = wg_off + N_WGS + 1
    n_items, n_split, n_wg, total = int(w[0]), int(w[1]), int(w[2]), int(w[3])
    G = case.num_q_heads // hkv
    assert list(w[4:16]) == [256 // G, 64, nqt, nkt, 0x32504342, case.batch, hkv, int(w[11]), 0,
                             int(case.q_blk is not None), case.total_q, case.max_pages_per_seq * case.page_size]
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


# ------------------------------------------------------------------ stale or foreign plans

def _plan_for(meta, nbytes=None):
    plan = torch.empty(nbytes or bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    bcp.build_tile_mask(meta, plan=plan)
    return plan


def _attn_with_plan(dc, meta, plan):
    out = torch.full_like(dc.q, float("nan"))
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    bcp.attn_block_causal_paged(meta, dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, out, plan=plan,
                                workspace=ws)
    torch.cuda.synchronize()
    return out


def test_checked_mode_rejects_a_plan_of_another_step():
    case = small_case(61, G=4, d=128, D=16, P=16)
    other = small_case(62, G=4, d=128, D=16, P=16, batch=4)
    dc, do = DeviceCase(case), DeviceCase(other)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    meta_o = bcp.StepMeta(**do.meta_kwargs(), check=True)
    nbytes = max(bcp.plan_size(meta), bcp.plan_size(meta_o))
    # A plan built for another step shape.
    with pytest.raises(bcp.BcpError) as e:
        _attn_with_plan(dc, meta, _plan_for(meta_o, nbytes))
    assert e.value.code == bcp.BCP_E_ARG and "shape" in str(e.value)
    # A stale plan: the same shapes, but one committed length has moved since it was built.
    plan = _plan_for(meta)
    s = int(np.argmax(case.kv_len))
    kvl = dc.kv_len.clone()
    kvl[s] -= 1
    meta_stale = bcp.StepMeta(**{**dc.meta_kwargs(), "kv_len": kvl}, check=True)
    with pytest.raises(bcp.BcpError) as e:
        _attn_with_plan(dc, meta_stale, plan)
    assert e.value.code == bcp.BCP_E_ARG and "stale" in str(e.value)
    # Memory that build_tile_mask never wrote.
    with pytest.raises(bcp.BcpError) as e:
        _attn_with_plan(dc, meta, torch.zeros(bcp.plan_size(meta), dtype=torch.uint8, device="cuda"))
    assert e.value.code == bcp.BCP_E_ARG
    # The step's own plan passes, and gives the oracle's result.
    O_ref, _ = oracle_attention(case)
    assert_close(_attn_with_plan(dc, meta, plan), O_ref, "bf16", what="own plan")


def test_unchecked_kernels_ignore_a_plan_of_another_shape():
    """Without checked mode a plan of another shape reaches the kernels, which compare its
    header with their own arguments and do nothing: the output keeps its previous contents."""
    case = small_case(63, G=4, d=128, D=16, P=16)
    other = small_case(64, G=4, d=128, D=16, P=16, batch=5, max_kv=900)
    dc, do = DeviceCase(case), DeviceCase(other)
    meta = bcp.StepMeta(**dc.meta_kwargs())
    meta_o = bcp.StepMeta(**do.meta_kwargs())
    nbytes = max(bcp.plan_size(meta), bcp.plan_size(meta_o))
    out = _attn_with_plan(dc, meta, _plan_for(meta_o, nbytes))
    assert torch.isnan(out.float()).all()


# ------------------------------------------------------------------ promotion order -------

def promotion_order(case, rng):
    """Fixture: the same step with each sequence's committed rows -- keys, values, block ids
    and positions together -- moved to random slots among its own, and its live rows (with
    their ids and positions) interleaved at random. Block ids then follow no order in either
    region, as after promote-one-step-late and arena compaction ("Inference: Fewer, smaller
    forwards", Advancements 10 and 11), so most tiles are partial."""
    import copy
    c = copy.copy(case)
    P, Hkv, d = case.page_size, case.num_kv_heads, case.head_dim
    c.k_cache, c.v_cache = case.k_cache.copy(), case.v_cache.copy()
    c.kv_blk = case.kv_blk.copy()
    c.kv_pos = None if case.kv_pos is None else case.kv_pos.copy()
    c.q, c.k_new, c.v_new, c.q_blk = case.q.copy(), case.k_new.copy(), case.v_new.copy(), case.q_blk.copy()
    c.q_pos = None if case.q_pos is None else case.q_pos.copy()
    kc, vc = c.k_cache.reshape(-1, Hkv, d), c.v_cache.reshape(-1, Hkv, d)
    k0, v0 = case.k_cache.reshape(-1, Hkv, d), case.v_cache.reshape(-1, Hkv, d)
    for s in range(case.batch):
        n = int(case.kv_len[s])
        j = np.arange(n)
        slots = case.page_table[s, j // P].astype(np.int64) * P + j % P
        src = slots[rng.permutation(n)]
        kc[slots], vc[slots], c.kv_blk[slots] = k0[src], v0[src], case.kv_blk[src]
        if c.kv_pos is not None:
            c.kv_pos[slots] = case.kv_pos[src]
        lo, hi = int(case.cu_q[s]), int(case.cu_q[s + 1])
        src = lo + rng.permutation(hi - lo)
        for name in ("q", "k_new", "v_new", "q_blk") + (("q_pos",) if c.q_pos is not None else ()):
            getattr(c, name)[lo:hi] = getattr(case, name)[src]
    return c


@pytest.mark.parametrize("window", [0, 512])
def test_C4_promotion_order(workloads, window):
    """C4 with every sequence's rows in promotion order, four sequences in full."""
    case = promotion_order(workloads(4), np.random.default_rng(4004))
    rows = {s: np.arange(int(case.q_lens[s])) for s in (0, 5, 10, 15)}
    kw = dict(window=window, q_pos=case.q_pos, kv_pos=case.kv_pos) if window else {}
    O_ref, L_ref = oracle_attention(case, rows=rows, **kw)
    dc = DeviceCase(case)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    out, lse = run_attn(dc, stats=stats, window=window)
    assert_close(out, O_ref, "bf16", lse, L_ref, what=f"C4 promotion order, window {window}")
    st = stats.cpu().numpy()
    say(f"  tiles full {st[0]} partial {st[1]} skipped {st[2]}")
    assert st[1] > st[0]     # the per-key mask does most of the work
