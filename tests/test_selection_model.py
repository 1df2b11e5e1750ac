"""A host model of the device's exact top-p threshold search, checked against the
oracle with the acceptance rule on large, tied and near-tied mass vectors.

The model restates the algorithm the index kernel runs in its last workgroup
(fp32 block masses, composite keys (mass bits, inverted block id), fixed-point
masses in 2^-62 units; at most 64 candidates above the pruning floor are ranked
exactly at once; otherwise a first 256-bin level of eighth-octave bins from the
floor (half-octave bins from 0 without one), then refinement by 256-bin histograms
over the mass bits while more than 64 candidates of unequal mass remain, exact ranking
of the rest, and the equal-mass case resolved by count in ascending block order).  It exercises the algorithm's logic at sizes and
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


def _level(bits, fm, lo, hi, shift, cab, P, floor=0):
    """One histogram level over the candidates in [lo, hi] (and >= floor): bin =
    min((bits - lo) >> shift, 255); returns (mass above, count, lo, hi) of the bin where
    the cumulative mass from the top reaches P, or None."""
    bm = [0] * BINS
    bc = [0] * BINS
    for b_, f in zip(bits, fm):
        if lo <= b_ <= hi and b_ >= floor:
            k = min((b_ - lo) >> shift, BINS - 1)
            bm[k] += f
            bc[k] += 1
    above = cab
    for k in range(BINS - 1, -1, -1):
        if bm[k] > 0 and above < P <= above + bm[k]:
            nlo = lo + (k << shift)
            nhi = hi if k == BINS - 1 else min(hi, nlo + (1 << shift) - 1)
            return above, bc[k], nlo, nhi
        above += bm[k]
    return None


def prune_floor(p: float, n: int) -> int:
    """Bits of the device's pruning floor (1 - p - 1e-6) / (2 n), in fp32 as the device
    computes it: blocks below it stay out of the histograms."""
    f32 = np.float32
    x = f32(0.5) * (f32(1.0) - f32(p) - f32(1e-6)) / f32(n)
    return int(np.array(max(f32(0.0), x), dtype=np.float32).view(np.uint32))


def model_select(m64, p, prune=True):
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
    # first level: over the blocks above the pruning floor, built in the same pass as the
    # masses
    floor = prune_floor(p, n) if prune else 0
    cand_all = [j for j in range(n) if bits[j] >= floor]
    if len(cand_all) <= FINAL:
        # few candidates: ranked exactly at once (no crossing: every block)
        run, thr = 0, None
        for j in sorted(cand_all, key=lambda j: keys[j], reverse=True):
            if run < P <= run + fm[j]:
                thr = keys[j]
                break
            run += fm[j]
        if thr is None:
            return np.arange(n), 0
        return np.array(sorted(j for j in cand_all if keys[j] >= thr)), 0
    shift1 = 20 if floor else 22     # eighth-octave bins from the floor, else half-octave from 0
    lo1 = floor & ~((1 << shift1) - 1)
    r = _level(bits, fm, lo1, 0xFFFFFFFF, shift1, 0, P, floor)
    if r is None:  # the total mass is below p
        assert sum(fm) < P
        return np.arange(n), 0
    cab, cnt, lo, hi = r
    lo = min(max(lo, floor), hi)
    levels = 1
    while cnt > FINAL and lo < hi:
        span = hi - lo
        shift = max(0, span.bit_length() - 8)
        assert (span >> shift) < BINS
        r = _level(bits, fm, lo, hi, shift, cab, P)
        assert r is not None
        ncab, nc, nlo, nhi = r
        assert nhi - nlo < span
        cab, cnt, lo, hi = ncab, nc, nlo, nhi
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
        # the compaction's count: blocks above the range plus the admitted candidates
        n_above = sum(1 for j in range(n) if bits[j] > hi)
        n_cand = sum(1 for j in cands if keys[j] >= thr)
        assert n_above + n_cand == sum(1 for j in range(n) if keys[j] >= thr)
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
    assert levels <= 4
    # pruning the negligible blocks never changes the set
    G0, _ = model_select(m, p, prune=False)
    assert np.array_equal(G, G0)


def test_model_ties_follow_block_order():
    m = np.full(3000, 1.0 / 3000)
    for p in (0.1, 0.5, 0.77):
        G, _ = model_select(m, p)
        k = int(np.ceil(np.float32(p) * 3000 - 1e-9))
        assert G.tolist() == list(range(len(G)))
        assert abs(len(G) - k) <= 1
