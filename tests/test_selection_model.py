"""A host model of the device's exact top-p threshold search, checked against the
oracle with the acceptance rule on large, tied and near-tied mass vectors.

The model restates the algorithm the index kernel runs in its last workgroup
(fp32 block masses, composite keys (mass bits, inverted block id), fixed-point
masses in 2^-62 units, splitter refinement while more than 512 candidates remain,
exact ranking of the rest).  It exercises the algorithm's logic at sizes and
distributions the device sees (up to 16384 blocks) without a GPU; the device code
itself is covered by the GPU parity tests.
"""
import numpy as np
import pytest

from oracle import accept as A
from oracle import rtp_oracle as O

SPLITTERS = 63
FINAL = 512
MASK64 = (1 << 64) - 1


def _keys(mf):
    bits = mf.astype(np.float32).view(np.uint32).astype(np.uint64)
    j = np.arange(mf.shape[0], dtype=np.uint64)
    return (bits << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - j)


def _fixed(mf):
    return [int(np.float64(x) * 2.0 ** 62) for x in mf.astype(np.float32)]


def model_select(m64, p):
    """Blocks the device algorithm selects for fp64 masses m64 and threshold p (fp32)."""
    mf = np.asarray(m64, dtype=np.float32)
    n = mf.shape[0]
    p = float(np.float32(p))
    if p >= 1.0 or n == 1:
        return np.arange(n), 0
    keys = [int(k) for k in _keys(mf)]
    fm = _fixed(mf)
    P = int(np.ceil(np.ldexp(p, 62)))
    if sum(fm) < P:
        return np.arange(n), 0
    lo, hi, cab, cnt = 1, MASK64, 0, n
    levels = 0
    while cnt > FINAL:
        cands = [j for j in range(n) if lo <= keys[j] < hi]
        assert len(cands) == cnt
        stride = cnt // SPLITTERS
        samp = [keys[cands[o]] for o in range(0, SPLITTERS * stride, stride)]
        split = sorted(samp, reverse=True)
        bc = [0] * (SPLITTERS + 1)
        bm = [0] * (SPLITTERS + 1)
        for j in cands:
            a = sum(1 for s in split if s > keys[j])
            bc[a] += 1
            bm[a] += fm[j]
        run = cab
        for b in range(SPLITTERS + 1):
            if run + bm[b] >= P and run < P:
                new = (bc[b], split[b - 1] if b > 0 else hi, split[b] if b < SPLITTERS else lo, run)
                break
            run += bm[b]
        nc, hi, lo, cab = new
        assert 0 < nc < cnt
        cnt = nc
        levels += 1
    cands = sorted((keys[j] for j in range(n) if lo <= keys[j] < hi), reverse=True)
    run = cab
    thr = None
    for k in cands:
        f = fm[MASK64 & (0xFFFFFFFF - (k & 0xFFFFFFFF))]
        if run < P <= run + f:
            thr = k
            break
        run += f
    assert thr is not None
    return np.array([j for j in range(n) if keys[j] >= thr]), levels


def _masses(kind, n, g):
    if kind == "diffuse":
        s = g.standard_normal(n) * 0.2
        s[g.choice(n, size=max(1, n // 10), replace=False)] += 2.0
    elif kind == "peaked":
        s = g.standard_normal(n) * 4.0
        s[g.integers(0, n)] += 40.0
    elif kind == "needles":
        s = g.standard_normal(n) * 3.0
        s[g.choice(n, size=8, replace=False)] = s.max() + 4.0
    elif kind == "flat":
        s = np.zeros(n)
    elif kind == "two_level":
        s = np.where(g.random(n) < 0.5, 0.0, np.log(2.0))
    else:
        raise ValueError(kind)
    e = np.exp(s - s.max())
    return e / e.sum()


CASES = [(kind, n, p) for kind in ("diffuse", "peaked", "needles", "flat", "two_level")
         for n, p in ((700, 0.9), (2048, 0.95), (4096, 0.99), (8192, 0.95), (16384, 0.9))]


@pytest.mark.parametrize("kind,n,p", CASES, ids=[f"{k}-{n}-{p}" for k, n, p in CASES])
def test_model_matches_oracle(kind, n, p):
    g = np.random.default_rng(n + int(p * 1000) + len(kind))
    m = _masses(kind, n, g)
    G, levels = model_select(m, p)
    sel = O.select_top_p(m, float(np.float32(p)))
    ok, why = A.accept_selection(m, float(np.float32(p)), G, sel)
    assert ok, why
    if kind in ("diffuse", "peaked") and n > FINAL:
        assert levels <= 3


def test_model_ties_follow_block_order():
    m = np.full(3000, 1.0 / 3000)
    for p in (0.1, 0.5, 0.77):
        G, _ = model_select(m, p)
        k = int(np.ceil(np.float32(p) * 3000 - 1e-9))
        assert G.tolist() == list(range(len(G)))
        assert abs(len(G) - k) <= 1
