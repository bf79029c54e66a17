"""The allocation-free attention entry point against the ordinary one.

attn_block_causal_paged_noalloc keeps its split-KV partials (and the plan, when none is
passed) in the library's static per-GPU scratch instead of a caller's workspace. Two calls
in a row -- a decode step whose key tiles are split across workgroups, then a smaller step
-- must each give the ordinary entry point's output and LSE bit for bit (the same kernels
run), and the oracle's within the parity bounds; with and without a prebuilt plan.
"""
import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
from tests.oracle_helpers import oracle_attention
from tests.test_gpu_parity import assert_close, say, small_case
from workloads import config
from workloads.device import DeviceCase

pytestmark = pytest.mark.gpu


def both(dc, with_plan):
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    plan = None
    if with_plan:
        plan = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
        bcp.build_tile_mask(meta, plan=plan)
    shape = tuple(dc.q.shape[:2])
    out = torch.full_like(dc.q, float("nan"))
    lse = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    bcp.attn_block_causal_paged(meta, dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, out, plan=plan, lse=lse,
                                workspace=ws)
    out_n = torch.full_like(dc.q, float("nan"))
    lse_n = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    bcp.attn_block_causal_paged_noalloc(meta, dc.q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, out_n, plan=plan,
                                        lse=lse_n, stats=stats)
    torch.cuda.synchronize()
    return out, lse, out_n, lse_n, stats


@pytest.mark.parametrize("with_plan", [True, False])
def test_noalloc_matches_the_workspace_call_twice(with_plan):
    big = config(2)                                      # 8 sequences, key tiles split over 256 workgroups
    small = small_case(141, dtype="bf16", G=4, d=128, D=16, P=16, batch=3, max_q=70, max_kv=900)
    for k, case in enumerate((big, small)):
        dc = DeviceCase(case)
        out, lse, out_n, lse_n, stats = both(dc, with_plan)
        say(f"call {k}: batch {case.batch}, plan {with_plan}, tiles {stats.cpu().numpy().tolist()}")
        assert torch.equal(out.view(torch.int16), out_n.view(torch.int16))
        assert torch.equal(lse, lse_n)
        O_ref, L_ref = oracle_attention(case)
        assert_close(out_n, O_ref, "bf16", lse_n, L_ref, what=f"noalloc call {k}")
        assert int(stats[0].item() + stats[1].item()) > 0
