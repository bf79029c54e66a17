"""GPU parity of narrow work items: short live blocks (at most 64 packed rows per sequence
and kv head), such as the short causal extend of "Introspective Diffusion Language Models"
(its serving section: 2N-1 causal query rows per step over the paged cache, one paged
kernel for extends of up to nine tokens).

For bf16 steps whose max_q_len * (Hq/Hkv) <= 64 the library picks q-tiles of 64/(Hq/Hkv)
positions and the two-wave narrow kernel; every case here checks that geometry was chosen
and compares with the oracle (and, with and without a plan, bit for bit with itself).
"""
import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
from tests.oracle_helpers import oracle_attention, oracle_tiles
from tests.test_gpu_parity import assert_close, check_tiles, run_attn, say, small_case
from tests.test_gpu_live_in_cache import place_live_rows
from workloads import config
from workloads.device import DeviceCase

pytestmark = pytest.mark.gpu


def narrow_q_tiles(dc):
    c = dc.case
    G = c.num_q_heads // c.num_kv_heads
    meta = bcp.StepMeta(**dc.meta_kwargs())
    return bcp.num_q_tiles(meta) == -(-c.max_q_len // (64 // G))


CASES = [
    dict(seed=81, G=4, d=128, D=1, P=16, max_q=9, max_kv=900, batch=6),      # the extend shape
    dict(seed=82, G=4, d=128, D=4, P=16, max_q=16, max_kv=300),
    dict(seed=83, G=8, d=128, D=1, P=12, max_q=8, max_kv=700, batch=5),
    dict(seed=84, G=2, d=64, D=3, P=8, max_q=32, max_kv=500),
    dict(seed=85, G=1, d=128, D=16, P=64, max_q=64, max_kv=1300),
    dict(seed=86, G=16, d=64, D=1, P=3, max_q=4, max_kv=200, batch=7),
    dict(seed=87, G=4, d=128, D=1, P=16, mode="B", max_q=16, max_kv=600),
    dict(seed=88, G=4, d=64, D=1, P=32, max_q=9, max_kv=5000, batch=4),       # long caches, split items
    dict(seed=94, G=8, d=64, D=1, P=16, max_q=8, max_kv=2500, batch=9),       # several items per workgroup
    # block ids in promotion order (no order among live or committed rows)
    dict(seed=92, G=4, d=128, D=1, P=16, mode="Bu", max_q=16, max_kv=600),
    dict(seed=93, G=16, d=64, D=1, P=8, mode="Bu", max_q=4, max_kv=3000, batch=5),
]


@pytest.mark.parametrize("spec", CASES, ids=lambda s: "-".join(f"{k}{v}" for k, v in s.items()))
def test_narrow_small(spec):
    case = small_case(dtype="bf16", **spec)
    say(f"narrow case {spec}: q_lens {case.q_lens.tolist()} kv_lens {case.kv_len.tolist()}")
    dc = DeviceCase(case)
    assert narrow_q_tiles(dc)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="narrow")
    out2, _ = run_attn(dc, plan=False, want_lse=False)
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))


def test_narrow_tile_classes_and_plan():
    case = small_case(89, dtype="bf16", G=4, d=128, D=1, P=16, max_q=9, max_kv=900, batch=6)
    check_tiles(case, 16, 64, with_plan=True)


def test_narrow_window_and_live_rows_in_cache():
    case = small_case(90, dtype="bf16", G=4, d=128, D=1, P=16, max_q=9, max_kv=1500, batch=6)
    dc = DeviceCase(case)
    assert narrow_q_tiles(dc)
    O_ref, L_ref = oracle_attention(case, window=300)
    out, lse = run_attn(dc, window=300)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="narrow, window 300")
    kc, vc = place_live_rows(case, dc)
    v = type("V", (), {})()
    v.__dict__.update(dc.__dict__)
    v.meta_kwargs, v.k_cache, v.v_cache, v.k_new, v.v_new = dc.meta_kwargs, kc, vc, None, None
    out_ip, lse_ip = run_attn(v, live_in_cache=True, window=300)
    assert torch.equal(out.view(torch.uint8), out_ip.view(torch.uint8)) and torch.equal(lse, lse_ip)


def test_narrow_poisoned_pages():
    # Slots past kv_len in each sequence's last page hold NaN (as unmapped pages do): the
    # ragged tails of narrow items must never bring them into a visible score.
    case = small_case(91, dtype="bf16", G=4, d=128, D=1, P=16, max_q=9, max_kv=400, batch=5)
    for s in range(case.batch):
        n = int(case.kv_len[s])
        for j in range(n, -(-n // 16) * 16):
            pg = case.page_table[s, j // 16]
            case.k_cache[pg, j % 16] = 0x7FC0
            case.v_cache[pg, j % 16] = 0x7FC0
    dc = DeviceCase(case)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="narrow poisoned")


def test_C6_short_causal_extend_full():
    case = config(6)
    dc = DeviceCase(case)
    assert narrow_q_tiles(dc)
    O_ref, L_ref = oracle_attention(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, "bf16", lse, L_ref, what="C6")
    np.testing.assert_array_equal(check_tiles(case, 16, 64, with_plan=True), oracle_tiles(case, 16, 64))
