"""Step graphs on the GPU: a captured step (tile classification and plan, two attention
layers, KV commit) replayed several times, with the program's own work and
synchronizations between the replays, reproduces the eager step bit for bit."""
import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
from workloads import config
from workloads.device import DeviceCase

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def test_graph_replays_match_eager():
    case = config(2)
    dc = DeviceCase(case)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=False)
    nqt, nkt = bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)
    plan = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    tc = torch.empty((case.batch, nqt, nkt), dtype=torch.uint8, device="cuda")
    q2 = (dc.q.float() * 0.5).to(dc.q.dtype).contiguous()     # a second layer's queries
    total = int(case.total_q)

    def outputs():
        o = [torch.empty_like(dc.q) for _ in range(2)]
        l = [torch.empty(tuple(dc.q.shape[:2]), dtype=torch.float32, device="cuda") for _ in range(2)]
        return o, l

    def step(o, l):
        bcp.build_tile_mask(meta, tile_class=tc, plan=plan)
        for q, oo, ll in ((dc.q, o[0], l[0]), (q2, o[1], l[1])):
            bcp.attn_block_causal_paged(meta, q, dc.k_new, dc.v_new, dc.k_cache, dc.v_cache, oo, plan=plan,
                                        lse=ll, workspace=ws)
        bcp.kv_commit_block(meta, dc.k_new, dc.v_new, dc.cu_q, dc.kv_len, dc.k_cache, dc.v_cache, total)

    s = torch.cuda.Stream()
    eo, el = outputs()
    with torch.cuda.stream(s):
        step(eo, el)
    s.synchronize()
    e_tc, e_k, e_v = tc.cpu().numpy(), bits(dc.k_cache), bits(dc.v_cache)

    go, gl = outputs()
    with torch.cuda.stream(s):
        bcp.graph_begin(s)
        step(go, gl)
        graph = bcp.graph_end(s)
    try:
        for rep in range(3):
            for t in go + gl:        # the program's own work between replays
                t.fill_(float("nan"))
            tc.fill_(255)
            torch.cuda.synchronize()
            graph.launch(s)
            s.synchronize()
            for a, b in zip(go, eo):
                np.testing.assert_array_equal(bits(a), bits(b))
            for a, b in zip(gl, el):
                np.testing.assert_array_equal(bits(a), bits(b))
            np.testing.assert_array_equal(tc.cpu().numpy(), e_tc)
            np.testing.assert_array_equal(bits(dc.k_cache), e_k)
            np.testing.assert_array_equal(bits(dc.v_cache), e_v)
    finally:
        graph.close()


def test_checked_mode_refused_under_capture():
    case = config(1)
    dc = DeviceCase(case)
    meta = bcp.StepMeta(**dc.meta_kwargs(), check=True)
    plan = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bcp.graph_begin(s)
        with pytest.raises(bcp.BcpError):
            bcp.build_tile_mask(meta, plan=plan)
        graph = bcp.graph_end(s)     # the capture holds nothing
    graph.launch(s)
    s.synchronize()
    graph.close()
