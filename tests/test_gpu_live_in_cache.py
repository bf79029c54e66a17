"""GPU parity of the in-place layout: live keys and values already in the cache pool.

With BCP_F_LIVE_IN_CACHE the active block's keys and values sit in the pool at logical
rows kv_len + i (the producer wrote them there), attention reads one paged source, and
committing them only moves block ids ("Inference: Fewer, smaller forwards", Advancement
11). The fixture below places the live rows into their slots through the page table; the
result must match the oracle (which takes the live rows separately: the definition does
not depend on where they are stored) and be bit-identical to the library's own path with
separate live rows, since every tile holds the same values either way.
"""
import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
import oracle
from tests.oracle_helpers import oracle_attention
from tests.test_gpu_parity import assert_close, run_attn, say, small_case
from workloads import config, make_case
from workloads.device import DeviceCase, to_host_bits

pytestmark = pytest.mark.gpu


def live_slots(case):
    """(page, slot) of every live row when it sits at logical row kv_len + i (fixture)."""
    pages, slots = [], []
    for s in range(case.batch):
        n, k = int(case.cu_q[s + 1] - case.cu_q[s]), int(case.kv_len[s])
        j = k + np.arange(n)
        pages.append(case.page_table[s, j // case.page_size])
        slots.append(j % case.page_size)
    return np.concatenate(pages + [np.zeros(0, np.int64)]), np.concatenate(slots + [np.zeros(0, np.int64)])


def place_live_rows(case, dc):
    """Pools holding the committed rows and, at kv_len + i, the live rows."""
    pg, sl = live_slots(case)
    assert (pg >= 0).all(), "fixture needs pages mapped for the live rows"
    pg = torch.from_numpy(pg.astype(np.int64)).cuda()
    sl = torch.from_numpy(sl.astype(np.int64)).cuda()
    kc, vc = dc.k_cache.clone(), dc.v_cache.clone()
    kc[pg, sl] = dc.k_new
    vc[pg, sl] = dc.v_new
    return kc, vc


def run_in_place(dc, kc, vc, plan=True, check=True):
    class View:   # the same device case with the in-place pools
        pass
    v = View()
    v.__dict__.update(dc.__dict__)
    v.meta_kwargs = dc.meta_kwargs
    v.k_cache, v.v_cache = kc, vc
    v.k_new = v.v_new = None
    return run_attn(v, plan=plan, check=check, live_in_cache=True)


def same_bits(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


CASES = [
    dict(seed=61, dtype="bf16", G=4, d=128, D=16, P=16),
    dict(seed=62, dtype="bf16", G=4, d=128, D=64, P=64, batch=5, max_q=300, max_kv=700),
    dict(seed=63, dtype="bf16", G=2, d=64, D=3, P=12),       # runs cross pages; kv_len unaligned
    dict(seed=64, dtype="bf16", G=8, d=128, D=1, P=3),
    dict(seed=65, dtype="bf16", G=4, d=128, D=1, P=16, mode="B"),
    dict(seed=66, dtype="bf16", G=4, d=64, D=1, P=8, mode="B", max_q=200, max_kv=900),
    dict(seed=67, dtype="f32", G=4, d=128, D=16, P=16),
    dict(seed=68, dtype="f32", G=2, d=64, D=1, P=8, mode="B"),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_live_rows_in_cache_small(spec):
    case = small_case(**spec)
    say(f"in-place case {spec}: q_lens {case.q_lens.tolist()} kv_lens {case.kv_len.tolist()}")
    dc = DeviceCase(case)
    kc, vc = place_live_rows(case, dc)
    out, lse = run_in_place(dc, kc, vc)
    O_ref, L_ref = oracle_attention(case)
    assert_close(out, O_ref, case.dtype, lse, L_ref, what="in place")
    sep, sep_lse = run_attn(dc)
    assert same_bits(out, sep) and torch.equal(lse, sep_lse)
    out2, _ = run_in_place(dc, kc, vc, plan=False, check=False)
    assert same_bits(out, out2)


def test_live_rows_in_cache_window():
    case = small_case(69, G=4, d=128, D=16, P=16, batch=4, max_q=130, max_kv=500)
    dc = DeviceCase(case)
    kc, vc = place_live_rows(case, dc)
    v = type("V", (), {})()
    v.__dict__.update(dc.__dict__)
    v.meta_kwargs, v.k_cache, v.v_cache, v.k_new, v.v_new = dc.meta_kwargs, kc, vc, None, None
    out, lse = run_attn(v, live_in_cache=True, window=37)
    O_ref, L_ref = oracle_attention(case, window=37)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="in place, window 37")


@pytest.mark.parametrize("n", [2, 4])
def test_live_rows_in_cache_workloads(n):
    case = config(n)
    dc = DeviceCase(case)
    kc, vc = place_live_rows(case, dc)
    out, lse = run_in_place(dc, kc, vc, check=True)
    sep, sep_lse = run_attn(dc, check=False)
    assert same_bits(out, sep) and torch.equal(lse, sep_lse)
    if n == 2:
        O_ref, L_ref = oracle_attention(case)
        assert_close(out, O_ref, "bf16", lse, L_ref, what=f"C{n} in place")


@pytest.mark.parametrize("mode", ["A", "B"])
def test_in_place_commit_moves_only_block_ids(mode):
    case = small_case(70 if mode == "A" else 71, G=4, d=64, D=8, P=16, mode=mode)
    dc = DeviceCase(case)
    kc, vc = place_live_rows(case, dc)
    kbits, vbits = to_host_bits(kc), to_host_bits(vc)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True, live_in_cache=True)
    kv_blk = dc.kv_blk.clone() if dc.kv_blk is not None else None
    bcp.kv_commit_block(meta, None, None, dc.cu_q, dc.kv_len, kc, vc, case.total_q,
                        src_blk=dc.q_blk, kv_blk_out=kv_blk, n_src=case.total_q)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(kc), kbits) and np.array_equal(to_host_bits(vc), vbits)
    if mode == "B":
        _, _, ref_blk = oracle.commit(case.k_cache, case.v_cache, case.k_new, case.v_new, case.cu_q,
                                      case.kv_len, case.page_table, case.page_size, case.num_pages,
                                      kv_blk=case.kv_blk, src_blk=case.q_blk)
        np.testing.assert_array_equal(kv_blk.cpu().numpy(), ref_blk)


def test_in_place_checked_mode_rejects_unmapped_live_rows():
    rng = np.random.default_rng(72)
    case = make_case(72, dtype="bf16", num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
                     page_size=16, q_lens=[20, 30], kv_lens=[40, 16], room_rows=[0, 30], rng=rng)
    dc = DeviceCase(case)
    out = torch.empty_like(dc.q)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True, live_in_cache=True)
    with pytest.raises(bcp.BcpError) as e:
        bcp.attn_block_causal_paged(meta, dc.q, None, None, dc.k_cache, dc.v_cache, out,
                                    workspace=torch.empty(bcp.attn_workspace_size(meta), dtype=torch.uint8,
                                                          device="cuda"))
    assert e.value.code == bcp.BCP_E_RANGE
