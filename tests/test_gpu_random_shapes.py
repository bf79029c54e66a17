"""GPU parity on shapes drawn at random (hypothesis, derandomized so every run draws the same
examples): block size D in {1, 2, 3, 16, 64, 256}, page size in {16, 32, 64} and odd sizes,
committed lengths including 0, 1 and lengths just off a page or tile edge, 1 to 5 sequences
(some with no live rows), GQA groups 1/2/4/8/16, head_dim 64/128, modes A, B (sorted ids) and
B in promotion order, bf16 and float32, permuted pages, and NaN in every slot past a
sequence's committed rows. Each example is checked against the oracle to the parity bounds,
and bit for bit with and without a prebuilt plan.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests.oracle_helpers import oracle_attention
from tests.test_gpu_parity import assert_close, run_attn, say
from workloads import BF16_NAN, make_case
from workloads.device import DeviceCase

pytestmark = pytest.mark.gpu


def poison_tails(case):
    """NaN in the slots past each sequence's committed rows in its mapped pages."""
    nan = BF16_NAN if case.dtype == "bf16" else np.float32(np.nan)
    P = case.page_size
    for s in range(case.batch):
        n = int(case.kv_len[s])
        for j in range(n, int((case.page_table[s] >= 0).sum()) * P):
            pg = case.page_table[s, j // P]
            case.k_cache[pg, j % P] = nan
            case.v_cache[pg, j % P] = nan


@st.composite
def shapes(draw):
    P = draw(st.sampled_from([16, 32, 64, 16, 32, 64, 1, 5, 24]))
    batch = draw(st.integers(1, 5))
    edge = st.sampled_from([0, 1, P - 1, P, P + 1, 63, 64, 65, 127, 129])
    kv = draw(st.lists(st.one_of(edge, st.integers(0, 700)), min_size=batch, max_size=batch))
    q = draw(st.lists(st.one_of(st.integers(0, 12), st.integers(0, 160)), min_size=batch, max_size=batch))
    if sum(q) == 0:
        q[draw(st.integers(0, batch - 1))] = draw(st.integers(1, 40))
    return dict(
        D=draw(st.sampled_from([1, 2, 3, 16, 64, 256])), P=P,
        G=draw(st.sampled_from([1, 2, 4, 8, 16])), Hkv=draw(st.sampled_from([1, 2, 3])),
        d=draw(st.sampled_from([64, 128])), mode=draw(st.sampled_from(["A", "A", "B", "Bu"])),
        dtype=draw(st.sampled_from(["bf16", "bf16", "bf16", "f32"])), q_lens=q, kv_lens=kv,
        seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=60, derandomize=True, deadline=None, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(shapes())
def test_random_shapes(spec):
    rng = np.random.default_rng(spec["seed"])
    d, G, Hkv = spec["d"], spec["G"], spec["Hkv"]
    kw = {}
    if spec["mode"] != "A":
        qb = [rng.integers(1, 6, n) for n in spec["q_lens"]]
        kb = [rng.integers(0, 6, n) for n in spec["kv_lens"]]
        if spec["mode"] == "B":
            qb, kb = [np.sort(b) for b in qb], [np.sort(b) for b in kb]
        kw = dict(q_blk_seqs=qb, kv_blk_seqs=kb)
    case = make_case(spec["seed"], dtype=spec["dtype"], num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                     block_size=spec["D"] if spec["mode"] == "A" else 1, page_size=spec["P"],
                     q_lens=spec["q_lens"], kv_lens=spec["kv_lens"], qkv_std=1 / np.sqrt(d), rng=rng, **kw)
    poison_tails(case)
    say(f"random shape {spec}")
    O_ref, L_ref = oracle_attention(case)
    dc = DeviceCase(case)
    out, lse = run_attn(dc)
    assert_close(out, O_ref, case.dtype, lse, L_ref, what="random shape")
    out2, _ = run_attn(dc, plan=False, want_lse=False)
    same = (torch.equal(out.view(torch.uint8), out2.view(torch.uint8)) if out.dtype == torch.bfloat16
            else torch.equal(out, out2))
    assert same
