"""Seeded synthetic inputs for block-causal paged attention.

This module only draws and lays out inputs: sequence lengths, block ids, page
tables, and the random Q/K/V values. It holds no attention, masking, tiling,
translation or commit arithmetic, so both the CPU oracle and the GPU path can
consume its output without sharing any of the method's code.

Layouts (all row-major, numpy):
  q        [total_q, Hq, d]      live query rows of the active blocks
  k_new    [total_q, Hkv, d]     live keys of the active blocks (RoPE already in)
  v_new    [total_q, Hkv, d]
  k_cache  [num_pages, P, Hkv, d] paged pool of committed keys
  v_cache  [num_pages, P, Hkv, d]
  cu_q     [batch+1] int32       live-row offsets per sequence
  kv_len   [batch]   int32       committed rows per sequence
  page_table [batch, max_pages_per_seq] int32, -1 where no page is mapped
  q_blk    [total_q] int32 or None           block id per live row (mode B)
  kv_blk   [num_pages*P] int32 or None       block id per cache slot (mode B)

bf16 tensors are carried as uint16 bit patterns; fp32 tensors as float32.
Unused cache pages (and pages mapped only as room for the next commit) hold
the NaN sentinel, so a kernel that reads them poisons its output.

Generation order for one seed (PCG64): structure and lengths, then the page
permutation, then Q, k_new, v_new, cached K, cached V.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs are finite (drawn from a normal distribution), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


@dataclasses.dataclass
class Case:
    name: str
    dtype: str                  # "bf16" or "f32"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int             # D (mode A); ignored by the mask in mode B
    page_size: int
    num_pages: int
    cu_q: np.ndarray
    kv_len: np.ndarray
    page_table: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q_blk: Optional[np.ndarray] = None
    kv_blk: Optional[np.ndarray] = None
    desc: str = ""
    # Mode B structure in logical row order, per sequence (what the page placement used).
    q_blk_seqs: Optional[list] = None
    kv_blk_seqs: Optional[list] = None
    # Absolute positions (multi-canvas layout), when the workload has them: per live row and
    # per cache slot (unused slots hold a position far from every row).
    q_pos: Optional[np.ndarray] = None
    kv_pos: Optional[np.ndarray] = None

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_q)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_len.max()) if self.batch else 0

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def mode(self) -> str:
        return "B" if self.q_blk is not None else "A"


def _normal(rng: np.random.Generator, shape, std: float, dtype: str, chunk_rows: int = 1 << 22):
    """Draw N(0, std^2) in float32, scale in float32, and store as `dtype` (bf16 bits or float32)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    std32 = np.float32(std)
    for lo in range(0, n, chunk_rows):
        hi = min(n, lo + chunk_rows)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= std32
        out[lo:hi] = bf16_bits(x) if dtype == "bf16" else x
    return out.reshape(shape)


def _nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, BF16_NAN, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def make_case(
    seed: int,
    *,
    name: str = "case",
    dtype: str = "bf16",
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    page_size: int,
    q_lens: Sequence[int],
    kv_lens: Sequence[int],
    num_pages: Optional[int] = None,
    pool_factor: float = 1.25,
    room_rows: Optional[Sequence[int]] = None,
    q_blk_seqs: Optional[Sequence[Sequence[int]]] = None,
    kv_blk_seqs: Optional[Sequence[Sequence[int]]] = None,
    identity_pages: bool = False,
    qkv_std: float = 1.0,
    rng: Optional[np.random.Generator] = None,
    desc: str = "",
) -> Case:
    """Build one case.

    q_lens/kv_lens: live and committed rows per sequence.
    room_rows: extra rows of mapped pages per sequence beyond kv_len (room for the
      next commit); defaults to q_lens.
    num_pages: pool size; default ceil(pool_factor * pages mapped).
    q_blk_seqs/kv_blk_seqs: per-sequence block-id lists (mode B), in logical row order.
    identity_pages: map pages 0,1,2,... in order instead of a random permutation.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    batch = len(q_lens)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    room = q_lens if room_rows is None else np.asarray(room_rows, dtype=np.int64)
    P = page_size
    mapped = [int(-(-(int(kv_lens[s]) + int(room[s])) // P)) for s in range(batch)]
    cached_pages = [int(-(-int(kv_lens[s]) // P)) for s in range(batch)]
    total_mapped = sum(mapped)
    if num_pages is None:
        num_pages = max(1, int(math.ceil(pool_factor * total_mapped)))
    assert num_pages >= total_mapped, "pool smaller than the pages the sequences map"
    maxp = max(1, max(mapped) if batch else 1)

    perm = np.arange(num_pages) if identity_pages else rng.permutation(num_pages)
    page_table = np.full((batch, maxp), -1, dtype=np.int32)
    nxt = 0
    for s in range(batch):
        page_table[s, : mapped[s]] = perm[nxt : nxt + mapped[s]]
        nxt += mapped[s]

    cu_q = np.zeros(batch + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    total_q = int(cu_q[-1])
    Hq, Hkv, d = num_q_heads, num_kv_heads, head_dim

    q = _normal(rng, (total_q, Hq, d), qkv_std, dtype)
    k_new = _normal(rng, (total_q, Hkv, d), qkv_std, dtype)
    v_new = _normal(rng, (total_q, Hkv, d), qkv_std, dtype)

    # Pages holding committed rows get random contents (every slot of the page);
    # everything else in the pool is NaN.
    holding = np.sort(np.concatenate(
        [page_table[s, : cached_pages[s]] for s in range(batch)] + [np.zeros(0, np.int32)]
    )).astype(np.int64)
    k_cache = _nan_fill((num_pages, P, Hkv, d), dtype)
    v_cache = _nan_fill((num_pages, P, Hkv, d), dtype)
    if holding.size:
        k_cache[holding] = _normal(rng, (holding.size, P, Hkv, d), qkv_std, dtype)
        v_cache[holding] = _normal(rng, (holding.size, P, Hkv, d), qkv_std, dtype)

    q_blk = kv_blk = None
    if q_blk_seqs is not None or kv_blk_seqs is not None:
        assert q_blk_seqs is not None and kv_blk_seqs is not None
        q_blk = np.concatenate([np.asarray(b, dtype=np.int32) for b in q_blk_seqs] + [np.zeros(0, np.int32)])
        assert q_blk.size == total_q
        # Block ids live beside the cached rows, page by page: sequence s's logical
        # rows [k*P, (k+1)*P) sit in its k-th mapped page. Slots past kv_len keep -1.
        kv_blk = np.full(num_pages * P, -1, dtype=np.int32).reshape(num_pages, P)
        for s in range(batch):
            ids = np.asarray(kv_blk_seqs[s], dtype=np.int32)
            assert ids.size == kv_lens[s]
            padded = np.full(cached_pages[s] * P, -1, dtype=np.int32)
            padded[: ids.size] = ids
            kv_blk[page_table[s, : cached_pages[s]]] = padded.reshape(cached_pages[s], P)
        kv_blk = kv_blk.reshape(-1)

    return Case(
        name=name, dtype=dtype, batch=batch, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        block_size=int(block_size), page_size=P, num_pages=int(num_pages), cu_q=cu_q,
        kv_len=kv_lens.astype(np.int32), page_table=page_table, q=q, k_new=k_new, v_new=v_new,
        k_cache=k_cache, v_cache=v_cache, q_blk=q_blk, kv_blk=kv_blk, desc=desc,
        q_blk_seqs=None if q_blk is None else [np.asarray(b, np.int32) for b in q_blk_seqs],
        kv_blk_seqs=None if q_blk is None else [np.asarray(b, np.int32) for b in kv_blk_seqs],
    )


# --------------------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-fp32: B1 2q/1kv d64 D16, 48 cached + 16 live, P16 identity pages",
    2: "steerling8b-decode: B8 32q/8kv d128 bf16 D64, kv U{512..4096 step 64}, P64 over a 4096-page pool",
    3: "prefill-commit: B4 32q/8kv d128 bf16, 8192-token prompt = 128 blocks of 64, P64 scattered",
    4: "multi-canvas: B16 32q/8kv d128 bf16, 1024 prompt + 3 canvases of 256, 30-100% live rows, P16",
    5: "long-context-decode: B64 32q/8kv d128 bf16 D64, kv lognormal clipped [1024,32768], P16",
    6: "short-causal-extend: B64 32q/8kv d128 bf16 D1, 9 live rows (5 for a quarter), kv U{64..3072}, P16",
}


def config(n: int, seed: Optional[int] = None) -> Case:
    """Synthetic stand-ins for the named workloads; seed defaults to 1000 + n."""
    seed = 1000 + n if seed is None else seed
    rng = np.random.default_rng(seed)
    inv = 1.0 / math.sqrt(128.0)
    if n == 1:
        return make_case(seed, name="C1", dtype="f32", num_q_heads=2, num_kv_heads=1, head_dim=64,
                         block_size=16, page_size=16, q_lens=[16], kv_lens=[48], num_pages=4,
                         identity_pages=True, qkv_std=1.0, rng=rng, desc=CONFIG_NAMES[1])
    if n == 2:
        kv = 64 * rng.integers(8, 65, size=8)
        return make_case(seed, name="C2", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                         block_size=64, page_size=64, q_lens=[64] * 8, kv_lens=kv, num_pages=4096,
                         qkv_std=inv, rng=rng, desc=CONFIG_NAMES[2])
    if n == 3:
        # 512 pages for the 4 x 8192 committed rows, plus one page each for the next block.
        return make_case(seed, name="C3", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                         block_size=64, page_size=64, q_lens=[8192] * 4, kv_lens=[0] * 4,
                         room_rows=[8192 + 64] * 4, num_pages=4096, qkv_std=1.0, rng=rng,
                         desc=CONFIG_NAMES[3])
    if n == 4:
        return _multi_canvas(seed, rng, inv)
    if n == 5:
        ln = rng.normal(math.log(4096.0), 1.0, size=64)
        kv = np.clip(np.floor(np.exp(ln)), 1024, 32768).astype(np.int64)
        return make_case(seed, name="C5", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                         block_size=64, page_size=16, q_lens=[64] * 64, kv_lens=kv, qkv_std=inv,
                         rng=rng, desc=CONFIG_NAMES[5])
    if n == 6:
        # Extend steps at concurrency 64: 2N-1 = 9 causal query rows per sequence (N = 5),
        # and N = 5 for a quarter of them (a proposal-only recovery step), over caches of
        # prompt plus generated tokens.
        ql = np.where(rng.random(64) < 0.25, 5, 9)
        kv = rng.integers(64, 3073, size=64)
        return make_case(seed, name="C6", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                         block_size=1, page_size=16, q_lens=ql, kv_lens=kv, qkv_std=inv, rng=rng,
                         desc=CONFIG_NAMES[6])
    raise ValueError(f"unknown config {n}")


def multi_canvas_structure(rng: np.random.Generator, batch: int, prompt: int, canvas: int,
                           n_canvas: int, lo: float = 0.3, hi: float = 1.0):
    """Per sequence: live rows are a random subset (fraction U[lo,hi]) of each canvas.

    Block ids: prompt = 0, canvas i = i (1-based). Committed rows are laid out prompt
    first, then each canvas's committed rows in canvas order; live rows in canvas order.
    Returns (q_lens, kv_lens, q_blk_seqs, kv_blk_seqs, live_positions, committed_positions).
    """
    q_lens, kv_lens, qb, kb, live_pos, com_pos = [], [], [], [], [], []
    for _ in range(batch):
        q_ids, k_ids = [], [0] * prompt
        lp, cp = [], list(range(prompt))
        for i in range(1, n_canvas + 1):
            f = rng.uniform(lo, hi)
            n_live = int(round(canvas * f))
            live = np.sort(rng.choice(canvas, size=n_live, replace=False))
            mask = np.ones(canvas, dtype=bool)
            mask[live] = False
            done = np.nonzero(mask)[0]
            base = prompt + (i - 1) * canvas
            q_ids += [i] * n_live
            k_ids += [i] * done.size
            lp += list(base + live)
            cp += list(base + done)
        q_lens.append(len(q_ids))
        kv_lens.append(len(k_ids))
        qb.append(q_ids)
        kb.append(k_ids)
        live_pos.append(lp)
        com_pos.append(cp)
    return q_lens, kv_lens, qb, kb, live_pos, com_pos


def _multi_canvas(seed: int, rng: np.random.Generator, std: float) -> Case:
    q_lens, kv_lens, qb, kb, live_pos, com_pos = multi_canvas_structure(rng, 16, 1024, 256, 3)
    case = make_case(seed, name="C4", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                     block_size=256, page_size=16, q_lens=q_lens, kv_lens=kv_lens, q_blk_seqs=qb,
                     kv_blk_seqs=kb, qkv_std=std, rng=rng, desc=CONFIG_NAMES[4])
    return with_positions(case, live_pos, com_pos)


def with_positions(case: Case, live_pos, com_pos) -> Case:
    """Attach q_pos [total_q] and kv_pos [num_pages*P]: committed row j of sequence s sits in
    page page_table[s, j//P], slot j%P, as its block id does."""
    case.q_pos = np.concatenate([np.asarray(p, np.int32) for p in live_pos] + [np.zeros(0, np.int32)])
    kv_pos = np.full(case.num_pages * case.page_size, -(10 ** 6), np.int32)
    for s, cp in enumerate(com_pos):
        for j, p in enumerate(cp):
            kv_pos[case.page_table[s, j // case.page_size] * case.page_size + j % case.page_size] = p
    case.kv_pos = kv_pos
    return case
