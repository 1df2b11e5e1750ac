"""Plain fp64 CPU oracle for RTPurbo's decode-time sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels.

Every function restates one definition from the pages, in fp64, with every bf16
input converted exactly.  Sources (page title, section):

* Review = the Korean paper review of RTPurbo on dongryeollee1.github.io,
  "Method" part.  Its "Adaptive sparse attention" equation defines the low-rank
  pre-RoPE index score s_h(m, n) = (W^Q_h q^pre_{m,h})^T (W^K_h k^pre_{n,h}) and
  the active set S_h(m) = Top-P(s_h(m, .), p); the same paragraph gives the
  local heads' sliding window + attention sink rule.  Its "Hardware-aware top-p
  decoding kernel" paragraph makes the top-p *block-wise* (a block mask found by
  a mass threshold).
* Strikes-Back = "Full Attention Strikes Back: Transferring Full Attention into
  Sparse within Hundred Training Steps" (aitrends.kr), numbered method item 2
  (low-rank retrieval routing): O_h(m) as a softmax of q^T k / sqrt(d_h) over
  S_h(m); its architecture paragraph names the cross-split reduce.

Readings taken where the pages are silent or garbled:

* Block mass = sum over the block's tokens of the softmax (over all N cached
  tokens of the sequence, current token included) of the raw index scores; no
  scale or temperature on the index score (neither formula has one).
* Greedy top-p: blocks by mass descending, ties by ascending block id; the
  smallest prefix whose cumulative mass reaches p; every block when no prefix
  does; p >= 1 selects every block.
* Static top-k (the Review's Experiments paragraph: a fixed-budget variant with
  k = 4096 built to isolate the dynamic budget; its Insight item 3 counts the
  budget in tokens): a budget of k tokens keeps ceil(k / block) blocks, the
  same order (mass descending, ties by ascending id); every block when the
  budget covers them.
* Strikes-Back's printed O_h(m) has lost its value vector; the output is the
  usual softmax(q K^T / sqrt(128)) V over the selected tokens.
* Retrieval heads attend to the selected tokens only (no forced sink/window).
* Local heads: tokens [0, min(S, N)) union [max(0, N - W), N), no double count.
* Cache append (the decode step before the path): the new token is the last of the
  N_b tokens (row N_b - 1); its index key for retrieval head h is W^K_h k^pre of
  the head's KV head, the exact dot products rounded once to bf16 (nearest, ties to
  even); its K and V rows are stored as given.
* Prefill (the Review's Adaptive sparse attention paragraph): causal; a local head's
  query at position i sees the decode rule's token set for N = i + 1, a retrieval
  head's sees every position up to i.  The prompt's index keys are each computed as
  in the cache append.

Parity of every function here is pinned by tests/test_oracle_pins.py (closed
forms, brute force, library routines, hand-worked golden fixtures).
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
INDEX_DIM = 16


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp64 (a bf16 value is the top half of an fp32 pattern)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- index (Kernel 1)
def bf16_round(x) -> int:
    """bf16 bit pattern of the real number x (a float or an exact Fraction), rounded
    once to nearest with ties to even: 8 significant bits, float32's exponent range,
    subnormals (quantum 2^-133) below 2^-126, infinity beyond the largest finite value."""
    if isinstance(x, float) and math.isnan(x):
        return 0x7FC0
    if isinstance(x, float) and math.isinf(x):
        return (0x8000 if x < 0 else 0) | 0x7F80
    neg = (x < 0) or (isinstance(x, float) and x == 0.0 and math.copysign(1.0, x) < 0)
    sign = 0x8000 if neg else 0
    a = abs(Fraction(x))
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    if a < Fraction(2) ** e:
        e -= 1
    elif a >= Fraction(2) ** (e + 1):
        e += 1                                                   # now 2^e <= a < 2^(e+1)
    if e < -126:
        return sign | round(a * Fraction(2) ** 133)              # 128 = the smallest normal
    n = round(a * Fraction(2) ** (7 - e))                        # in [128, 256], ties to even
    if n == 256:
        n, e = 128, e + 1
    if e + 127 >= 255:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | (n - 128)


def index_key(w_k_h: np.ndarray, k_pre: np.ndarray) -> np.ndarray:
    """k_idx = bf16(W^K_h k^pre): 16 dot products over 128 dims, each summed exactly
    (rationals) and rounded once (Review, Adaptive sparse attention equation: the key
    side of s_h(m, n)).  Returns uint16 bf16 bit patterns [16]."""
    w = bf16_to_f64(w_k_h).reshape(INDEX_DIM, HEAD_DIM)
    k = bf16_to_f64(k_pre).reshape(HEAD_DIM)
    out = np.zeros(INDEX_DIM, dtype=np.uint16)
    for i in range(INDEX_DIM):
        exact = sum((Fraction(float(w[i, d])) * Fraction(float(k[d])) for d in range(HEAD_DIM)), Fraction(0))
        out[i] = bf16_round(exact)
    return out


def index_query(w_q_h: np.ndarray, q_pre: np.ndarray) -> np.ndarray:
    """q_idx = W^Q_h q^pre  (Review, Adaptive sparse attention equation).

    w_q_h: bf16 bits [16, 128]; q_pre: bf16 bits [128].  Returns fp64 [16].
    """
    W = bf16_to_f64(w_q_h)
    x = bf16_to_f64(q_pre)
    return W @ x


def index_scores(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """s_n = q_idx . k_idx_n for every cached token n (same equation).

    k_idx: bf16 bits [N, 16] holding W^K_h k^pre_n.  Returns fp64 [N].
    """
    return bf16_to_f64(k_idx) @ np.asarray(q_idx, dtype=np.float64)


def token_softmax(s: np.ndarray) -> np.ndarray:
    """Softmax of the index scores over all N tokens (max subtracted)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def block_masses(s: np.ndarray, block: int) -> np.ndarray:
    """m_j = sum of token probabilities over block j = [j*Bk, min((j+1)*Bk, N)).

    The block-wise mass behind the Review's block mask; the last block may be partial.
    """
    P = token_softmax(s)
    n = P.shape[0]
    nblk = -(-n // block)
    padded = np.zeros(nblk * block, dtype=np.float64)
    padded[:n] = P
    return padded.reshape(nblk, block).sum(axis=1)


@dataclasses.dataclass
class Selection:
    blocks: np.ndarray      # selected block ids, ascending (int64)
    order: np.ndarray       # all block ids by (mass desc, id asc)
    k_star: int             # number of selected blocks
    tau: float              # mass of the last admitted block (the threshold)
    c_prev: float           # cumulative mass before the last admitted block
    c_star: float           # cumulative mass including it
    all_blocks: bool        # p >= 1 or no prefix reached p


def select_top_p(m: np.ndarray, p: float) -> Selection:
    """Greedy block top-p: Top-P(s_h(m, .), p) at block granularity.

    Blocks in descending mass, ties by ascending id; keep the shortest prefix whose
    cumulative mass is >= p (Review, Adaptive sparse attention equation and the
    kernel paragraph's "cumulative mass reaches p_top" threshold).
    """
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    assert n >= 1
    assert p > 0.0, "top-p must be positive"
    ids = np.arange(n)
    order = np.lexsort((ids, -m))          # primary: -m ascending, secondary: id ascending
    csum = np.cumsum(m[order])
    if p >= 1.0:
        k = n
        all_blocks = True
    else:
        hit = np.nonzero(csum >= p)[0]
        if hit.size:
            k = int(hit[0]) + 1
            all_blocks = False
        else:
            k = n
            all_blocks = True
    blocks = np.sort(order[:k])
    tau = float(m[order[k - 1]])
    c_star = float(csum[k - 1])
    c_prev = float(csum[k - 2]) if k >= 2 else 0.0
    return Selection(blocks=blocks, order=order, k_star=k, tau=tau, c_prev=c_prev,
                     c_star=c_star, all_blocks=all_blocks)


def select_top_k(m: np.ndarray, k_tokens: int, block: int) -> Selection:
    """Static top-k at block granularity: a budget of k_tokens keeps the
    ceil(k_tokens / block) blocks of largest mass, ties by ascending id (Review,
    Experiments: the static top-k variant, k = 4096; Insight item 3: a fixed k
    counted in tokens); every block when there are no more than that."""
    m = np.asarray(m, dtype=np.float64)
    n = m.shape[0]
    assert n >= 1
    assert k_tokens >= 1 and block >= 1
    kb = -(-int(k_tokens) // int(block))
    ids = np.arange(n)
    order = np.lexsort((ids, -m))
    k = min(kb, n)
    csum = np.cumsum(m[order])
    blocks = np.sort(order[:k])
    return Selection(blocks=blocks, order=order, k_star=k, tau=float(m[order[k - 1]]),
                     c_prev=float(csum[k - 2]) if k >= 2 else 0.0, c_star=float(csum[k - 1]),
                     all_blocks=k == n)


def block_tokens(blocks: Sequence[int], block: int, n: int) -> np.ndarray:
    """Token ids of the given blocks, ascending, clipped to the context length."""
    out = [np.arange(j * block, min(n, (j + 1) * block)) for j in sorted(int(b) for b in blocks)]
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


# ------------------------------------------------------------ attention (Kernel 2)
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, tokens: np.ndarray) -> Tuple[np.ndarray, float]:
    """Exact softmax(q K^T / sqrt(128)) V over the given tokens (Strikes-Back O_h(m)).

    q: bf16 bits [128]; K, V: bf16 bits [T, 128] (the cache rows of one KV head);
    tokens: int token ids.  Returns (o fp64 [128], lse) with lse the natural log of
    sum_n exp(q.k_n / sqrt(128)).  An empty token set gives (0, -inf).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size == 0:
        return np.zeros(HEAD_DIM, dtype=np.float64), float("-inf")
    qf = bf16_to_f64(q)
    Kf = bf16_to_f64(K[tokens])
    Vf = bf16_to_f64(V[tokens])
    logits = (Kf @ qf) / np.sqrt(HEAD_DIM)
    mx = logits.max()
    w = np.exp(logits - mx)
    z = w.sum()
    return (w @ Vf) / z, float(mx + np.log(z))


def merge_partials(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, float]:
    """Cross-split reduce (Strikes-Back architecture paragraph).

    L = log sum_c exp(lse_c); o = sum_c exp(lse_c - L) o_c; empty parts have
    lse = -inf and weight 0.
    """
    lse = np.asarray(lse_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    live = np.isfinite(lse)
    if not live.any():
        return np.zeros(o.shape[-1]), float("-inf")
    mx = lse[live].max()
    w = np.where(live, np.exp(np.where(live, lse, mx) - mx), 0.0)
    L = mx + np.log(w.sum())
    return (w[:, None] * o).sum(axis=0) / w.sum(), float(L)


def local_tokens(n: int, window: int, sinks: int) -> np.ndarray:
    """Sliding window + attention sink token set (Review, Adaptive sparse attention).

    [0, min(S, N)) union [max(0, N - W), N), ascending, no duplicates.
    """
    return np.union1d(np.arange(min(sinks, n)), np.arange(max(0, n - window), n)).astype(np.int64)


# -------------------------------------------------------------------- decode step
@dataclasses.dataclass
class HeadResult:
    out: np.ndarray                  # fp64 [128]
    lse: float
    tokens: np.ndarray               # attended token ids
    masses: Optional[np.ndarray] = None      # retrieval heads: block masses
    selection: Optional[Selection] = None    # retrieval heads


def retrieval_head(inp, b: int, r: int) -> HeadResult:
    """Full oracle for one (sequence, retrieval head): index, top-p, exact attention."""
    cfg = inp.cfg
    n = int(inp.seq_lens[b])
    hq = int(inp.ret_heads[r])
    kv = hq // (cfg.Hq // cfg.Hkv)
    qi = index_query(inp.w_q[r], inp.q_pre[b, hq])
    s = index_scores(qi, inp.k_idx[b, r, :n])
    m = block_masses(s, cfg.block)
    sel = select_top_p(m, float(inp.top_p[b, r]))
    toks = block_tokens(sel.blocks, cfg.block, n)
    o, lse = attend(inp.q[b, hq], inp.k_cache[b, kv], inp.v_cache[b, kv], toks)
    return HeadResult(out=o, lse=lse, tokens=toks, masses=m, selection=sel)


def retrieval_masses(inp, b: int, r: int) -> np.ndarray:
    n = int(inp.seq_lens[b])
    hq = int(inp.ret_heads[r])
    qi = index_query(inp.w_q[r], inp.q_pre[b, hq])
    return block_masses(index_scores(qi, inp.k_idx[b, r, :n]), inp.cfg.block)


def local_head(inp, b: int, hq: int) -> HeadResult:
    """Full oracle for one (sequence, local head): window + sink exact attention."""
    cfg = inp.cfg
    n = int(inp.seq_lens[b])
    kv = hq // (cfg.Hq // cfg.Hkv)
    toks = local_tokens(n, cfg.window, cfg.sinks)
    o, lse = attend(inp.q[b, hq], inp.k_cache[b, kv], inp.v_cache[b, kv], toks)
    return HeadResult(out=o, lse=lse, tokens=toks)


def dense_head(inp, b: int, hq: int) -> HeadResult:
    """Dense decode attention over every cached token (for the p = 1 checks)."""
    cfg = inp.cfg
    n = int(inp.seq_lens[b])
    kv = hq // (cfg.Hq // cfg.Hkv)
    toks = np.arange(n)
    o, lse = attend(inp.q[b, hq], inp.k_cache[b, kv], inp.v_cache[b, kv], toks)
    return HeadResult(out=o, lse=lse, tokens=toks)


def decode_step(inp, items: Optional[Sequence[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], HeadResult]:
    """Oracle outputs for (b, query head) items (default: every head of every sequence)."""
    cfg = inp.cfg
    ret_index = {int(h): i for i, h in enumerate(inp.ret_heads)}
    if items is None:
        items = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    res = {}
    for b, h in items:
        if h in ret_index:
            res[(b, h)] = retrieval_head(inp, b, ret_index[h])
        else:
            res[(b, h)] = local_head(inp, b, h)
    return res


# ------------------------------------------------------------------------ prefill
def prefill_tokens(i: int, retrieval: bool, window: int, sinks: int) -> np.ndarray:
    """Keys the query at prompt position i attends to during prefill.

    Review, Adaptive sparse attention: local heads apply the sliding window + sink rule
    in prefill as in decode, and retrieval heads run full dense attention in prefill;
    Review, Efficiency & ultra-long robustness: prefill sparsity is fixed in advance
    (local heads see only sink 4 + window 8192).  Prefill is causal, so position i sees
    positions 0..i: the decode rule with N = i + 1 tokens (all of them for a retrieval
    head, local_tokens(i + 1, W, S) for a local head).
    """
    n = i + 1
    if retrieval:
        return np.arange(n, dtype=np.int64)
    return local_tokens(n, window, sinks)


def prefill_row(q_i: np.ndarray, K: np.ndarray, V: np.ndarray, i: int, retrieval: bool, window: int,
                sinks: int) -> Tuple[np.ndarray, float]:
    """Prefill output (fp64 [128], lse) of the query at position i: exact attention over
    prefill_tokens(i, ...).  q_i: bf16 bits [128]; K, V: bf16 bits [>= i + 1, 128], the
    prompt's rows of the head's KV group (row n = position n)."""
    return attend(q_i, K, V, prefill_tokens(i, retrieval, window, sinks))


def prefill_head(pin, b: int, hq: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Prefill outputs (fp64 [len(rows), 128]) of query head hq of sequence b for the
    given prompt positions (default: all N_b of them).  pin carries q [B, Hq, T, 128],
    k, v [B, Hkv, T, 128] (bf16 bits), seq_lens, ret_heads and the config's window,
    sinks and head counts; the head's KV group is hq // (Hq / Hkv)."""
    cfg = pin.cfg
    n = int(pin.seq_lens[b])
    kv = hq // (cfg.Hq // cfg.Hkv)
    ret = hq in {int(h) for h in pin.ret_heads}
    if rows is None:
        rows = range(n)
    return np.stack([prefill_row(pin.q[b, hq, i], pin.k[b, kv], pin.v[b, kv], int(i), ret, cfg.window,
                                 cfg.sinks)[0] for i in rows])
