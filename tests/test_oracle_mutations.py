"""The oracle pins catch plausible mistakes: each case plants one mistake in a copy of the
oracle (a comparison off by one, a transposed mask or operand, a wrong head mapping,
scale, log base, slot or page, a missing normalization or tile class) and checks that the
CPU pin suite fails on it. CPU only; each case runs the pins once in a subprocess.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (oracle file, original text, mistaken text, what the mistake is)
MUTS = [
    ("mask.py", "M[:, kv_len:] = (i[None, :] // D) <= (i[:, None] // D)", "M[:, kv_len:] = (i[None, :] // D) < (i[:, None] // D)", "mode A live <= -> <"),
    ("mask.py", "M[:, kv_len:] = (i[None, :] // D) <= (i[:, None] // D)", "M[:, kv_len:] = (i[:, None] // D) <= (i[None, :] // D)", "mode A live transposed"),
    ("mask.py", "M[:, kv_len:] = (i[None, :] // D) <= (i[:, None] // D)", "M[:, kv_len:] = (i[None, :] // D) <= (i[:, None] // D) + 1", "mode A sees next block"),
    ("mask.py", "M[:, :kv_len] = True", "M[:, :kv_len] = True; M[:, kv_len - 1:kv_len] = False", "mode A drops last committed key"),
    ("mask.py", "M[:, :kv_len] = kb[None, :] <= qb[:, None]", "M[:, :kv_len] = kb[None, :] < qb[:, None]", "mode B cached <= -> <"),
    ("mask.py", "M[:, kv_len:] = qb[None, :] <= qb[:, None]", "M[:, kv_len:] = qb[None, :] < qb[:, None]", "mode B live <= -> <"),
    ("mask.py", "M[:, kv_len:] = qb[None, :] <= qb[:, None]", "M[:, kv_len:] = qb[:, None] <= qb[None, :]", "mode B live transposed"),
    ("mask.py", "return M & ((qp[:, None] - kp[None, :]) < W)", "return M & ((qp[:, None] - kp[None, :]) <= W)", "window < -> <="),
    ("mask.py", "qp = kv_len + np.arange(q_len, dtype=np.int64)", "qp = np.arange(q_len, dtype=np.int64)", "window mode A positions"),
    ("attention.py", "Qg = Q[:, g * G:(g + 1) * G, :]", "Qg = Q[:, g::Hkv, :]", "GQA interleaved heads"),
    ("attention.py", "scale = 1.0 / np.sqrt(d) if scale is None else float(scale)", "scale = 1.0 / d if scale is None else float(scale)", "default scale 1/d"),
    ("attention.py", "Lg = np.where(ok, m_safe + np.log(l), -np.inf)", "Lg = np.where(ok, m_safe + np.log2(l), -np.inf)", "LSE log2"),
    ("attention.py", "Og = np.where(ok[:, :, None], Og / l[:, :, None], 0.0)", "Og = np.where(ok[:, :, None], Og, 0.0)", "no normalization"),
    ("attention.py", "Vf = np.concatenate([widen(v_cache[page, slot]), widen(v_new[lo:hi])], axis=0)", "Vf = np.concatenate([widen(k_cache[page, slot]), widen(v_new[lo:hi])], axis=0)", "K used as cached V"),
    ("attention.py", "Vf = np.concatenate([widen(v_cache[page, slot]), widen(v_new[lo:hi])], axis=0)", "Vf = np.concatenate([widen(v_cache[page, slot]), widen(v_new[lo:hi])[::-1]], axis=0)", "live V reversed"),
    ("attention.py", "Q = widen(q[lo + r])", "Q = widen(q[lo + r[::-1]]) if r.size > 1 else widen(q[lo + r])", "query rows reversed"),
    ("attention.py", "w = np.exp(S - m_safe[:, :, None])", "w = np.exp(S - m_safe[:, :, None]) * (1 + 1e-3)", "P scaled (cancels)"),
    ("paging.py", "return page, j % P", "return page, (j + 1) % P", "slot off by one"),
    ("paging.py", "page = page_table[s, logical_page].astype(np.int64)", "page = page_table[0, logical_page].astype(np.int64)", "page table row 0"),
    ("tiles.py", "out[s, r] = np.where(allv, TILE_FULL, np.where(anyv, TILE_PARTIAL, TILE_SKIP))", "out[s, r] = np.where(anyv, TILE_FULL, TILE_SKIP)", "no PARTIAL class"),
    ("tiles.py", "sub = grid[r * tq:min((r + 1) * tq, q_len)]", "sub = grid[r * tq:min((r + 1) * tq + 1, q_len)]", "q-tile one row too tall"),
]


@pytest.mark.parametrize("fn, old, new, name", MUTS, ids=[m[3] for m in MUTS])
def test_pins_catch_a_planted_mistake(fn, old, new, name):
    d = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        for x in ("tests", "workloads", "oracle"):
            shutil.copytree(os.path.join(ROOT, x), os.path.join(d, x),
                            ignore=shutil.ignore_patterns("__pycache__"))
        p = os.path.join(d, "oracle", fn)
        s = open(p).read()
        assert s.count(old) == 1, "the text to mutate is not in the oracle (oracle changed?)"
        open(p, "w").write(s.replace(old, new, 1))
        r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                            "-p", "no:cacheprovider"], cwd=d, capture_output=True, text=True, timeout=300)
        assert r.returncode != 0, f"the pins pass with the mistake '{name}' planted:\n{r.stdout[-2000:]}"
    finally:
        shutil.rmtree(d, ignore_errors=True)
