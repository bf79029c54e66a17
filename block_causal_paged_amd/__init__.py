"""Block-causal paged attention and KV commit on MI355X (gfx950).

Thin Python binding of libbcp.so (include/bcp.h): it only marshals arguments. Tensors
are torch device tensors; their memory and the current stream are handed to the C ABI,
and every step of the computation runs in the library's HIP kernels. There is no CPU
fallback: if the library is not built, every call raises.

Entry points (same names as the C ABI):
  build_tile_mask(meta, tile_class=None, phys_page=None, plan=None)
  attn_block_causal_paged(meta, q, k_new, v_new, k_cache, v_cache, out, plan=None, ...)
  attn_block_causal_paged_noalloc(meta, q, k_new, v_new, k_cache, v_cache, out, plan=None, ...)
  kv_commit_block(meta, k_src, v_src, cu_src, dst_start, k_cache, v_cache, total_commit, ...)
  graph_begin(stream), graph_end(stream) -> Graph, Graph.launch(stream), Graph.close()
    (bcp_graph_begin / _end / _launch / _destroy: capture a step's calls and replay them)
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbcp.so")

BCP_BF16, BCP_F32 = 0, 1
BCP_TILE_SKIP, BCP_TILE_PARTIAL, BCP_TILE_FULL = 0, 1, 2
BCP_OK, BCP_E_ARG, BCP_E_UNSUPPORTED, BCP_E_RANGE, BCP_E_WORKSPACE, BCP_E_HIP = range(6)
BCP_F_CHECK = 1
BCP_F_LIVE_IN_CACHE = 2

STATUS_NAMES = {0: "BCP_OK", 1: "BCP_E_ARG", 2: "BCP_E_UNSUPPORTED", 3: "BCP_E_RANGE",
                4: "BCP_E_WORKSPACE", 5: "BCP_E_HIP"}

# Every function include/bcp.h declares.
EXPORTED = ["bcp_num_q_tiles", "bcp_num_k_tiles", "bcp_plan_size", "build_tile_mask",
            "attn_block_causal_paged_workspace_size", "attn_block_causal_paged",
            "attn_block_causal_paged_noalloc", "kv_commit_block",
            "bcp_last_error", "bcp_abi_version", "bcp_graph_begin", "bcp_graph_end", "bcp_graph_launch",
            "bcp_graph_destroy"]


class BcpError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


class bcp_meta(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("cu_q", ctypes.c_void_p),
        ("q_blk", ctypes.c_void_p),
        ("total_q", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("kv_len", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("kv_blk", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("tile_q", ctypes.c_int32),
        ("tile_k", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("window", ctypes.c_int32),
        ("q_pos", ctypes.c_void_p),
        ("kv_pos", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded libbcp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, VP = ctypes.POINTER(bcp_meta), ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        L.bcp_abi_version.restype = ctypes.c_int
        L.bcp_last_error.restype = ctypes.c_char_p
        for n in ("bcp_num_q_tiles", "bcp_num_k_tiles"):
            getattr(L, n).argtypes, getattr(L, n).restype = [P], I32
        for n in ("bcp_plan_size", "attn_block_causal_paged_workspace_size"):
            getattr(L, n).argtypes, getattr(L, n).restype = [P], SZ
        L.build_tile_mask.argtypes = [P, VP, VP, VP, SZ, VP]
        L.build_tile_mask.restype = ctypes.c_int
        L.attn_block_causal_paged.argtypes = [P, VP, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP, VP, SZ, VP, VP]
        L.attn_block_causal_paged.restype = ctypes.c_int
        L.attn_block_causal_paged_noalloc.argtypes = [P, VP, VP, VP, VP, VP, VP, ctypes.c_float, VP, VP, VP, VP]
        L.attn_block_causal_paged_noalloc.restype = ctypes.c_int
        L.kv_commit_block.argtypes = [P, VP, VP, VP, VP, VP, VP, I32, I32, VP, VP, VP, VP]
        L.kv_commit_block.restype = ctypes.c_int
        L.bcp_graph_begin.argtypes, L.bcp_graph_begin.restype = [VP], ctypes.c_int
        L.bcp_graph_end.argtypes, L.bcp_graph_end.restype = [VP, ctypes.POINTER(VP)], ctypes.c_int
        L.bcp_graph_launch.argtypes, L.bcp_graph_launch.restype = [VP, VP], ctypes.c_int
        L.bcp_graph_destroy.argtypes, L.bcp_graph_destroy.restype = [VP], None
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, ref):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    dev = ref.device if hasattr(ref, "device") and ref.device.type == "cuda" else None
    return torch.cuda.current_stream(dev).cuda_stream


def _check(rc):
    if rc != BCP_OK:
        raise BcpError(rc, lib().bcp_last_error().decode())


class StepMeta:
    """bcp_meta for one step plus references to the device metadata it points at.

    cu_q, kv_len, page_table (and q_blk/kv_blk in mode B) are int32 device tensors;
    total_q, max_q_len and max_kv_len are the host-side bounds the C ABI asks for.
    """

    def __init__(self, *, dtype, batch, num_q_heads, num_kv_heads, head_dim, block_size, cu_q,
                 kv_len, page_table, num_pages, page_size, total_q, max_q_len, max_kv_len,
                 q_blk=None, kv_blk=None, tile_q=0, tile_k=0, check=False, window=0,
                 live_in_cache=False, q_pos=None, kv_pos=None):
        self._refs = (cu_q, kv_len, page_table, q_blk, kv_blk, q_pos, kv_pos)
        self.device_ref = cu_q
        self.c = bcp_meta(
            struct_size=ctypes.sizeof(bcp_meta),
            dtype=BCP_BF16 if dtype in ("bf16", BCP_BF16) else BCP_F32,
            batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
            block_size=block_size, cu_q=_ptr(cu_q), q_blk=_ptr(q_blk), total_q=total_q,
            max_q_len=max_q_len, kv_len=_ptr(kv_len), page_table=_ptr(page_table),
            kv_blk=_ptr(kv_blk), num_pages=num_pages, page_size=page_size,
            max_pages_per_seq=int(page_table.shape[1]) if hasattr(page_table, "shape") else 1,
            max_kv_len=max_kv_len, tile_q=tile_q, tile_k=tile_k, flags=(BCP_F_CHECK if check else 0) | (BCP_F_LIVE_IN_CACHE if live_in_cache else 0),
            window=int(window or 0), q_pos=_ptr(q_pos), kv_pos=_ptr(kv_pos),
        )

    @property
    def ref(self):
        return ctypes.byref(self.c)


def num_q_tiles(meta):
    return lib().bcp_num_q_tiles(meta.ref)


def num_k_tiles(meta):
    return lib().bcp_num_k_tiles(meta.ref)


def plan_size(meta):
    return lib().bcp_plan_size(meta.ref)


def attn_workspace_size(meta):
    return lib().attn_block_causal_paged_workspace_size(meta.ref)


def build_tile_mask(meta, tile_class=None, phys_page=None, plan=None, stream=None):
    nbytes = 0 if plan is None else plan.numel() * plan.element_size()
    _check(lib().build_tile_mask(meta.ref, _ptr(tile_class), _ptr(phys_page), _ptr(plan), nbytes,
                                 _stream(stream, meta.device_ref)))


def attn_block_causal_paged(meta, q, k_new, v_new, k_cache, v_cache, out, plan=None, scale=0.0,
                            lse=None, workspace=None, stats=None, stream=None):
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_block_causal_paged(meta.ref, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                         _ptr(v_cache), _ptr(plan), float(scale), _ptr(out), _ptr(lse),
                                         _ptr(workspace), wbytes, _ptr(stats), _stream(stream, q)))


NOALLOC_SCRATCH_BYTES = 76 << 20    # BCP_NOALLOC_SCRATCH_BYTES


def attn_block_causal_paged_noalloc(meta, q, k_new, v_new, k_cache, v_cache, out, plan=None, scale=0.0,
                                    lse=None, stats=None, stream=None):
    """The allocation-free attention call: no workspace; the library's static per-GPU scratch
    holds the split partials (and the plan when `plan` is None)."""
    _check(lib().attn_block_causal_paged_noalloc(meta.ref, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                                 _ptr(v_cache), _ptr(plan), float(scale), _ptr(out), _ptr(lse),
                                                 _ptr(stats), _stream(stream, q)))


def kv_commit_block(meta, k_src, v_src, cu_src, dst_start, k_cache, v_cache, total_commit,
                    src_row=None, src_blk=None, kv_blk_out=None, n_src=None, stream=None):
    if n_src is None:
        n_src = int((k_src if k_src is not None else src_blk).shape[0])
    _check(lib().kv_commit_block(meta.ref, _ptr(k_src), _ptr(v_src), _ptr(cu_src), _ptr(src_row),
                                 _ptr(dst_start), _ptr(src_blk), int(total_commit), int(n_src),
                                 _ptr(k_cache), _ptr(v_cache), _ptr(kv_blk_out),
                                 _stream(stream, k_cache)))


def _graph_stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def graph_begin(stream=None):
    """Start capturing the calls made on `stream` (not the legacy default stream)."""
    _check(lib().bcp_graph_begin(_graph_stream(stream)))


class Graph:
    """A captured step (bcp_graph); launch() replays it, close() releases it."""

    def __init__(self, handle):
        self._h = handle

    def launch(self, stream=None):
        if not self._h:
            raise BcpError(BCP_E_ARG, "graph is closed")
        _check(lib().bcp_graph_launch(self._h, _graph_stream(stream)))

    def close(self):
        if self._h:
            lib().bcp_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def graph_end(stream=None):
    """End the capture started by graph_begin on `stream`; returns the instantiated Graph."""
    h = ctypes.c_void_p()
    _check(lib().bcp_graph_end(_graph_stream(stream), ctypes.byref(h)))
    return Graph(h.value)
