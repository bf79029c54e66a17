"""Step graphs on the GPU: a captured step replayed several times, with the program's own
work and synchronizations between the replays.

* A model step of 32 layers (the tile mask and plan built once, then every layer's attention
  call over its own queries and its own K/V pool, and every layer's KV commit) reproduces the
  oracle on every replay: each layer's output and LSE within the parity tolerance, each
  layer's pools bit for bit, the tile classes exactly.
* A C2 step (two attention layers) reproduces the eager step bit for bit.
"""
import copy

import numpy as np
import pytest
import torch

import block_causal_paged_amd as bcp
import oracle
from tests.oracle_helpers import oracle_attention, oracle_tiles
from tests.test_gpu_parity import assert_close, say, small_case
from workloads import BF16_NAN, _normal, config
from workloads.device import DeviceCase, to_host_bits

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


def layer_cases(base, n_layers, seed):
    """Per-layer inputs on one step structure: fresh Q, live K/V and committed K/V for every
    layer (same lengths, pages and unused NaN slots as `base`)."""
    rng = np.random.default_rng(seed)
    std = 1.0 / np.sqrt(base.head_dim)
    out = []
    for _ in range(n_layers):
        c = copy.copy(base)
        c.q = _normal(rng, base.q.shape, std, "bf16")
        c.k_new = _normal(rng, base.k_new.shape, std, "bf16")
        c.v_new = _normal(rng, base.v_new.shape, std, "bf16")
        for name in ("k_cache", "v_cache"):
            x = getattr(base, name).copy()
            live = x != BF16_NAN
            x[live] = _normal(rng, (int(live.sum()),), std, "bf16")
            setattr(c, name, x)
        out.append(c)
    return out


def test_graph_32_layer_step_matches_oracle():
    L = 32
    base = small_case(131, dtype="bf16", G=4, Hkv=2, d=128, D=16, P=16, batch=3, max_q=70, max_kv=300)
    layers = layer_cases(base, L, 132)
    dcs = [DeviceCase(c) for c in layers]
    meta = bcp.StepMeta(**dcs[0].meta_kwargs(), check=False)
    nqt, nkt = bcp.num_q_tiles(meta), bcp.num_k_tiles(meta)
    plan = torch.empty(bcp.plan_size(meta), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(1, bcp.attn_workspace_size(meta)), dtype=torch.uint8, device="cuda")
    tc = torch.empty((base.batch, nqt, nkt), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(d.q) for d in dcs]
    lses = [torch.empty(tuple(d.q.shape[:2]), dtype=torch.float32, device="cuda") for d in dcs]
    cu, dst = dcs[0].cu_q, dcs[0].kv_len

    refs = [oracle_attention(c) for c in layers]
    pools = [oracle.commit(c.k_cache, c.v_cache, c.k_new, c.v_new, c.cu_q, c.kv_len, c.page_table, c.page_size,
                           c.num_pages)[:2] for c in layers]
    ref_tc = oracle_tiles(base, 256 // 4, 64)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bcp.graph_begin(s)
        bcp.build_tile_mask(meta, tile_class=tc, plan=plan)
        for d, o, l in zip(dcs, outs, lses):
            bcp.attn_block_causal_paged(meta, d.q, d.k_new, d.v_new, d.k_cache, d.v_cache, o, plan=plan, lse=l,
                                        workspace=ws)
            bcp.kv_commit_block(meta, d.k_new, d.v_new, cu, dst, d.k_cache, d.v_cache, base.total_q)
        graph = bcp.graph_end(s)
    try:
        for rep in range(3):
            for t in outs + lses:     # the program's own work between replays
                t.fill_(float("nan"))
            tc.fill_(255)
            torch.cuda.synchronize()
            graph.launch(s)
            s.synchronize()
            say(f"replay {rep}")
            np.testing.assert_array_equal(tc.cpu().numpy(), ref_tc)
            for k, (o, l, (O_ref, L_ref), (kc, vc), d) in enumerate(zip(outs, lses, refs, pools, dcs)):
                assert_close(o, O_ref, "bf16", l, L_ref, what=f"layer {k}")
                np.testing.assert_array_equal(to_host_bits(d.k_cache), kc)
                np.testing.assert_array_equal(to_host_bits(d.v_cache), vc)
    finally:
        graph.close()
