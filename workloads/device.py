"""Copy a workloads.Case to the GPU as torch tensors (input plumbing; no method arithmetic)."""
import numpy as np
import torch


class DeviceCase:
    """Device copies of a Case's arrays plus the host-side bounds the C ABI needs."""

    def __init__(self, case, device="cuda"):
        self.case = case
        dev = torch.device(device)
        store = torch.bfloat16 if case.dtype == "bf16" else torch.float32

        def data(x):
            t = torch.from_numpy(np.ascontiguousarray(x))
            if case.dtype == "bf16":
                t = t.view(torch.int16).view(torch.bfloat16)   # same bits
            return t.to(dev)

        def ints(x):
            return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

        self.dtype = store
        self.q, self.k_new, self.v_new = data(case.q), data(case.k_new), data(case.v_new)
        self.k_cache, self.v_cache = data(case.k_cache), data(case.v_cache)
        self.cu_q, self.kv_len, self.page_table = ints(case.cu_q), ints(case.kv_len), ints(case.page_table)
        self.q_blk, self.kv_blk = ints(case.q_blk), ints(case.kv_blk)
        self.q_pos, self.kv_pos = ints(case.q_pos), ints(case.kv_pos)

    def meta_kwargs(self):
        c = self.case
        return dict(dtype=c.dtype, batch=c.batch, num_q_heads=c.num_q_heads,
                    num_kv_heads=c.num_kv_heads, head_dim=c.head_dim, block_size=c.block_size,
                    cu_q=self.cu_q, kv_len=self.kv_len, page_table=self.page_table,
                    num_pages=c.num_pages, page_size=c.page_size, total_q=c.total_q,
                    max_q_len=c.max_q_len, max_kv_len=c.max_kv_len, q_blk=self.q_blk,
                    kv_blk=self.kv_blk, q_pos=self.q_pos, kv_pos=self.kv_pos)


def to_host_bits(t):
    """Device tensor -> numpy array with the stored bits (uint16 for bf16, float32 for fp32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
