"""Host-side checks of the C ABI, runnable without a GPU.

The library must load and export every function include/bcp.h declares, and every
malformed host argument must be rejected with its status code before anything touches a
device (the pointers used here are fake, never dereferenced).
"""
import ctypes
import os
import re

import pytest

import block_causal_paged_amd as bcp

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "bcp.h")
FAKE = 0x10000   # a 64 KiB-aligned fake device address; validation only checks alignment


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_function():
    L = bcp.lib()
    decl = declared_functions()
    assert set(decl) == set(bcp.EXPORTED), decl
    for name in decl:
        assert hasattr(L, name), name
    assert L.bcp_abi_version() == 3


def meta(**over):
    kw = dict(struct_size=ctypes.sizeof(bcp.bcp_meta), dtype=bcp.BCP_BF16, batch=8, num_q_heads=32,
              num_kv_heads=8, head_dim=128, block_size=64, cu_q=FAKE, q_blk=None, total_q=512,
              max_q_len=64, kv_len=FAKE, page_table=FAKE, kv_blk=None, num_pages=4096, page_size=64,
              max_pages_per_seq=65, max_kv_len=4096, tile_q=0, tile_k=0, flags=0)
    kw.update(over)
    return bcp.bcp_meta(**kw)


def attn(m, workspace_bytes=1 << 40, **over):
    args = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, plan=FAKE, scale=0.0,
                out=FAKE, lse=None, ws=FAKE, wsb=workspace_bytes, stats=None)
    args.update(over)
    return bcp.lib().attn_block_causal_paged(ctypes.byref(m), args["q"], args["k_new"], args["v_new"],
                                             args["k_cache"], args["v_cache"], args["plan"],
                                             args["scale"], args["out"], args["lse"], args["ws"],
                                             args["wsb"], args["stats"], None)


def test_geometry_queries():
    m = meta()
    L = bcp.lib()
    assert L.bcp_num_q_tiles(ctypes.byref(m)) == 1          # 64 positions x 4 heads = 256 rows
    assert L.bcp_num_k_tiles(ctypes.byref(m)) == 64 + 1     # 4096/64 cached + 1 live
    assert L.bcp_plan_size(ctypes.byref(m)) > 0
    assert L.attn_block_causal_paged_workspace_size(ctypes.byref(m)) > 0
    assert L.bcp_plan_size(ctypes.byref(meta(struct_size=4))) == 0


@pytest.mark.parametrize("over,code", [
    (dict(struct_size=8), bcp.BCP_E_ARG),
    (dict(dtype=7), bcp.BCP_E_ARG),
    (dict(batch=0), bcp.BCP_E_ARG),
    (dict(num_q_heads=30), bcp.BCP_E_ARG),                # not a multiple of 8 kv heads
    (dict(cu_q=None), bcp.BCP_E_ARG),
    (dict(kv_len=FAKE + 2), bcp.BCP_E_ARG),               # misaligned metadata
    (dict(q_blk=FAKE), bcp.BCP_E_ARG),                    # mode B needs both id arrays
    (dict(block_size=0), bcp.BCP_E_ARG),
    (dict(page_size=0), bcp.BCP_E_ARG),
    (dict(total_q=513), bcp.BCP_E_ARG),                   # more than batch * max_q_len
    (dict(max_kv_len=65 * 64 + 1), bcp.BCP_E_ARG),        # beyond the page table's reach
    (dict(head_dim=96), bcp.BCP_E_UNSUPPORTED),
    (dict(num_q_heads=24), bcp.BCP_E_UNSUPPORTED),        # 3 query heads per kv head
    (dict(tile_q=32), bcp.BCP_E_UNSUPPORTED),
    (dict(tile_k=32), bcp.BCP_E_UNSUPPORTED),
    (dict(window=-1), bcp.BCP_E_ARG),
    (dict(flags=4), bcp.BCP_E_ARG),                       # unknown flag
    (dict(window=256, q_blk=FAKE, kv_blk=FAKE), bcp.BCP_E_ARG),     # window in mode B needs positions
    (dict(batch=1, total_q=64, max_pages_per_seq=1 << 21, page_size=2048, num_pages=16),
     bcp.BCP_E_ARG),                                       # 2^32 rows per sequence: past 32-bit rows
])
def test_attention_rejects_bad_meta(over, code):
    assert attn(meta(**over)) == code
    assert bcp.lib().bcp_last_error()


@pytest.mark.parametrize("over,code", [
    (dict(q=None), bcp.BCP_E_ARG),
    (dict(out=FAKE + 8), bcp.BCP_E_ARG),                  # misaligned tensor
    (dict(scale=float("nan")), bcp.BCP_E_ARG),
    (dict(wsb=16), bcp.BCP_E_WORKSPACE),
    (dict(plan=None, wsb=1024), bcp.BCP_E_WORKSPACE),     # building the plan needs room too
])
def test_attention_rejects_bad_buffers(over, code):
    assert attn(meta(), **over) == code


def test_live_rows_in_cache_need_no_separate_live_buffers():
    # Without the flag NULL live buffers are refused; with it they are not read, so the call
    # gets as far as the workspace check.
    assert attn(meta(), k_new=None, v_new=None) == bcp.BCP_E_ARG
    assert attn(meta(flags=bcp.BCP_F_LIVE_IN_CACHE), k_new=None, v_new=None, wsb=16) == bcp.BCP_E_WORKSPACE


def test_tile_mask_rejects():
    L = bcp.lib()
    m = meta()
    assert L.build_tile_mask(ctypes.byref(m), None, None, None, 0, None) == bcp.BCP_E_ARG
    assert L.build_tile_mask(ctypes.byref(m), None, None, FAKE, 64, None) == bcp.BCP_E_WORKSPACE
    assert L.build_tile_mask(ctypes.byref(meta(struct_size=1)), FAKE, None, None, 0, None) == bcp.BCP_E_ARG
    assert b"NULL" in L.bcp_last_error() or L.bcp_last_error()


def test_commit_rejects():
    L = bcp.lib()

    def commit(m, **over):
        a = dict(k_src=FAKE, v_src=FAKE, cu_src=FAKE, src_row=None, dst_start=FAKE, src_blk=None,
                 total=4, n_src=4, k_cache=FAKE, v_cache=FAKE, kv_blk_out=None)
        a.update(over)
        return L.kv_commit_block(ctypes.byref(m), a["k_src"], a["v_src"], a["cu_src"], a["src_row"],
                                 a["dst_start"], a["src_blk"], a["total"], a["n_src"], a["k_cache"],
                                 a["v_cache"], a["kv_blk_out"], None)

    assert commit(meta(struct_size=3)) == bcp.BCP_E_ARG
    assert commit(meta(), k_cache=None) == bcp.BCP_E_ARG
    assert commit(meta(), total=-1) == bcp.BCP_E_ARG
    assert commit(meta(), v_src=FAKE + 4) == bcp.BCP_E_ARG
    assert commit(meta(head_dim=4, num_kv_heads=1)) == bcp.BCP_E_UNSUPPORTED   # 8-byte rows
    assert commit(meta(), k_src=None) == bcp.BCP_E_ARG                         # one of the two
    assert commit(meta(), k_src=None, v_src=None) == bcp.BCP_OK                # no K/V and no tags: nothing
    inplace = meta(flags=bcp.BCP_F_LIVE_IN_CACHE)
    assert commit(inplace, k_src=None, v_src=None, src_blk=FAKE) == bcp.BCP_E_ARG   # ids need kv_blk_out
    assert commit(inplace, k_src=None, v_src=None) == bcp.BCP_OK              # mode A: nothing to move
    assert commit(meta(), total=0) == bcp.BCP_OK                              # nothing to do


def test_graph_entry_points_reject_null_handles():
    # Host-side checks only: no capture is started, so no GPU is needed.
    L = bcp.lib()
    assert L.bcp_graph_end(None, None) == bcp.BCP_E_ARG
    assert b"NULL" in L.bcp_last_error()
    assert L.bcp_graph_launch(None, None) == bcp.BCP_E_ARG
    L.bcp_graph_destroy(None)   # a no-op
    g = bcp.Graph(None)
    with pytest.raises(bcp.BcpError):
        g.launch(0)
    g.close()


def test_error_message_is_thread_local_and_specific():
    attn(meta(head_dim=96))
    assert b"head_dim 96" in bcp.lib().bcp_last_error()


def test_noalloc_rejects_a_step_beyond_its_scratch_before_any_hip_call():
    """The allocation-free call refuses a step whose scratch need (partials plus, with no plan,
    the plan) exceeds its static array, with BCP_E_WORKSPACE, before touching a device."""
    m = meta(max_q_len=100000, total_q=512)     # the plan's per-q-tile lists grow with the bound
    L = bcp.lib()
    need = L.bcp_plan_size(ctypes.byref(m))
    assert need > bcp.NOALLOC_SCRATCH_BYTES
    rc = L.attn_block_causal_paged_noalloc(ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.0, FAKE, None,
                                           None, None)
    assert rc == bcp.BCP_E_WORKSPACE
    assert b"allocation-free" in L.bcp_last_error()
    # Host-argument errors come first, as for the ordinary call.
    rc = L.attn_block_causal_paged_noalloc(ctypes.byref(meta(head_dim=96)), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                           0.0, FAKE, None, None, None)
    assert rc == bcp.BCP_E_UNSUPPORTED
