"""Acceptance rules for comparing a device result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see rtp_oracle.py).

Block sets.  Several block sets are correct when masses tie or nearly tie at the
threshold, or when a cumulative sum lands within rounding of p.  A device set G
is accepted against the oracle's fp64 masses m, threshold tau = m of the last
admitted block and cumulative mass C* at that block (eps = 1e-6) when:

* p >= 1: G is every block;
* otherwise all of
  R1  every block with m_j > tau + eps is in G;
  R2  every block in G has m_j >= tau - eps, or the crossing is ambiguous
      (C* - p <= eps) and m_j is within eps of the oracle's next-ranked block;
  R3  sum_{G} m >= p - eps            (coverage);
  R4  sum_{G} m - min_{G} m < p + eps (minimality).

Static top-k block sets (budget of kb = ceil(k / block) blocks) are accepted when G
has exactly min(kb, nblk) blocks, every block with m_j > tau + eps is in G and every
block in G has m_j >= tau - eps (tau = the oracle's kb-th largest mass).

Outputs.  max |g - o| <= 1e-2 and sum |g - o| / sum |o| <= 1e-3 over every
output element of a workload, with bf16 inputs and fp32 accumulation.
"""
from __future__ import annotations

from typing import Iterable, List, Tuple

import numpy as np

from .rtp_oracle import Selection, select_top_k, select_top_p

EPS_MASS = 1e-6
TOL_MAX_ABS = 1e-2
TOL_MEAN_REL = 1e-3


def accept_selection(m: np.ndarray, p: float, gpu_blocks: Iterable[int],
                     sel: Selection = None, eps: float = EPS_MASS) -> Tuple[bool, List[str]]:
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    G = np.asarray(sorted(int(j) for j in gpu_blocks), dtype=np.int64)
    why: List[str] = []
    if G.size != np.unique(G).size:
        why.append("duplicate block ids")
    if G.size and (G.min() < 0 or G.max() >= n):
        why.append("block id out of range")
    if why:
        return False, why
    if sel is None:
        sel = select_top_p(m, p)
    if p >= 1.0:
        if G.size != n:
            why.append(f"p>=1 must select all {n} blocks, got {G.size}")
        return not why, why
    inG = np.zeros(n, dtype=bool)
    inG[G] = True
    tau = sel.tau
    must = np.nonzero(m > tau + eps)[0]
    missing = must[~inG[must]]
    if missing.size:
        why.append(f"R1: {missing.size} blocks above tau+eps missing (e.g. {missing[:5].tolist()})")
    low = G[m[G] < tau - eps]
    if low.size:
        ok_extra = False
        if sel.c_star - p <= eps and sel.k_star < n:
            nxt = m[sel.order[sel.k_star]]
            ok_extra = bool(np.all(m[low] >= nxt - eps))
        if not ok_extra:
            why.append(f"R2: {low.size} blocks below tau-eps selected (e.g. {low[:5].tolist()})")
    tot = float(m[G].sum()) if G.size else 0.0
    if not sel.all_blocks and tot < p - eps:
        why.append(f"R3: coverage {tot!r} < p - eps")
    if G.size and tot - float(m[G].min()) >= p + eps:
        why.append(f"R4: not minimal: {tot!r} - {float(m[G].min())!r} >= p + eps")
    return not why, why


def accept_topk(m: np.ndarray, k_tokens: int, block: int, gpu_blocks: Iterable[int],
                sel: Selection = None, eps: float = EPS_MASS) -> Tuple[bool, List[str]]:
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    G = np.asarray(sorted(int(j) for j in gpu_blocks), dtype=np.int64)
    why: List[str] = []
    if G.size != np.unique(G).size:
        why.append("duplicate block ids")
    if G.size and (G.min() < 0 or G.max() >= n):
        why.append("block id out of range")
    if why:
        return False, why
    if sel is None:
        sel = select_top_k(m, k_tokens, block)
    if G.size != sel.k_star:
        why.append(f"size: {G.size} blocks, the budget keeps {sel.k_star}")
    inG = np.zeros(n, dtype=bool)
    inG[G] = True
    must = np.nonzero(m > sel.tau + eps)[0]
    missing = must[~inG[must]]
    if missing.size:
        why.append(f"{missing.size} blocks above tau+eps missing (e.g. {missing[:5].tolist()})")
    low = G[m[G] < sel.tau - eps]
    if low.size:
        why.append(f"{low.size} blocks below tau-eps selected (e.g. {low[:5].tolist()})")
    return not why, why


def output_errors(gpu: np.ndarray, ref: np.ndarray) -> Tuple[float, float]:
    """(max-abs, mean-rel) with mean-rel = sum|g - o| / sum|o|."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    d = np.abs(g - o)
    denom = float(np.abs(o).sum())
    return float(d.max()) if d.size else 0.0, float(d.sum() / denom) if denom > 0 else float(d.sum())


def outputs_ok(gpu: np.ndarray, ref: np.ndarray, max_abs: float = TOL_MAX_ABS,
               mean_rel: float = TOL_MEAN_REL) -> Tuple[bool, float, float]:
    ma, mr = output_errors(gpu, ref)
    ok = bool(np.all(np.isfinite(np.asarray(gpu)))) and ma <= max_abs and mr <= mean_rel
    return ok, ma, mr
