"""A host model of the device's exact top-p threshold search, checked against the
oracle with the acceptance rule on large, tied and near-tied mass vectors.

The model restates the algorithm the index kernel runs in its last workgroup
(fp32 block masses, composite keys (mass bits, inverted block id), fixed-point
masses in 2^-62 units, refinement by 256-bin histograms over the mass bits while
more than 64 candidates of unequal mass remain, exact ranking of the rest, and the
equal-mass case resolved by count in ascending block order).  It exercises the algorithm's logic at sizes and
distributions the device sees (up to 16384 blocks) without a GPU; the device code
itself is covered by the GPU parity tests.
"""
import numpy as np
import pytest

from oracle import accept as A
from oracle import rtp_oracle as O

BINS = 256
FINAL = 64
MASK64 = (1 << 64) - 1


def _fixed(mf):
    return [int(np.float64(x) * 2.0 ** 62) for x in mf.astype(np.float32)]


def model_select(m64, p):
    """Blocks the device algorithm selects for fp64 masses m64 and threshold p (fp32).

    Returns (blocks, levels)."""
    mf = np.asarray(m64, dtype=np.float32)
    n = mf.shape[0]
    p = float(np.float32(p))
    if p >= 1.0 or n == 1:
        return np.arange(n), 0
    bits = [int(b) for b in mf.view(np.uint32)]
    keys = [(bits[j] << 32) | (0xFFFFFFFF - j) for j in range(n)]
    fm = _fixed(mf)
    P = int(np.ceil(np.ldexp(p, 62)))
    if sum(fm) < P:
        return np.arange(n), 0
    lo, hi, cab, cnt = min(bits), max(bits), 0, n
    levels = 0
    while cnt > FINAL and lo < hi:
        span = hi - lo
        shift = max(0, span.bit_length() - 8)
        bm = [0] * BINS
        bc = [0] * BINS
        bmin = [None] * BINS
        bmax = [None] * BINS
        for j in range(n):
            if lo <= bits[j] <= hi:
                b = (bits[j] - lo) >> shift
                assert 0 <= b < BINS
                bm[b] += fm[j]
                bc[b] += 1
                bmin[b] = bits[j] if bmin[b] is None else min(bmin[b], bits[j])
                bmax[b] = bits[j] if bmax[b] is None else max(bmax[b], bits[j])
        above = cab
        for b in range(BINS - 1, -1, -1):
            if bm[b] > 0 and above < P <= above + bm[b]:
                new = (above, bc[b], bmin[b], bmax[b])
                break
            above += bm[b]
        cab, nc, nlo, nhi = new
        assert nhi - nlo < max(1, span) or span == 0
        cnt, lo, hi = nc, nlo, nhi
        levels += 1
    cands = [j for j in range(n) if lo <= bits[j] <= hi]
    assert len(cands) == cnt
    if cnt > FINAL:
        # all candidates have equal mass: the k-th in ascending block order
        f = fm[cands[0]]
        k = -(-(P - cab) // f)
        thr = keys[cands[k - 1]]
    else:
        run = cab
        thr = None
        for j in sorted(cands, key=lambda j: keys[j], reverse=True):
            if run < P <= run + fm[j]:
                thr = keys[j]
                break
            run += fm[j]
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
    assert levels <= 5


def test_model_ties_follow_block_order():
    m = np.full(3000, 1.0 / 3000)
    for p in (0.1, 0.5, 0.77):
        G, _ = model_select(m, p)
        k = int(np.ceil(np.float32(p) * 3000 - 1e-9))
        assert G.tolist() == list(range(len(G)))
        assert abs(len(G) - k) <= 1
