"""Plant plausible mistakes in the oracle (CPU only) and show a pin catches each.

Every mutant replaces one oracle function for the duration of one test; the
pins in test_oracle_pins.py must then fail.
"""
import numpy as np
import pytest

from oracle import rtp_oracle as O
import test_oracle_pins as P

_orig = {name: getattr(O, name) for name in
         ("block_masses", "token_softmax", "select_top_p", "select_top_k", "attend", "local_tokens",
          "bf16_round", "index_key",
          "merge_partials", "index_query", "retrieval_head", "prefill_tokens")}


def _masses_per_block_softmax(s, block):
    s = np.asarray(s, np.float64)
    n = s.shape[0]
    out = []
    for j in range(-(-n // block)):
        blk = s[j * block:(j + 1) * block]
        e = np.exp(blk - blk.max())
        out.append((e / e.sum()).sum() / (-(-n // block)))
    return np.array(out)


def _masses_drop_partial(s, block):
    P_ = _orig["token_softmax"](s)
    nfull = P_.shape[0] // block
    return P_[:nfull * block].reshape(nfull, block).sum(axis=1)


def _softmax_wrong_sign(s):
    s = np.asarray(s, np.float64)
    e = np.exp(s.max() - s)
    return e / e.sum()


def _select_generic(m, p, tie_desc=False, strict=False, extra=0):
    m = np.asarray(m, np.float64)
    n = m.shape[0]
    ids = np.arange(n)
    order = np.lexsort(((-ids if tie_desc else ids), -m))
    cs = np.cumsum(m[order])
    hit = np.nonzero(cs > p if strict else cs >= p)[0]
    k = n if (p >= 1.0 or not hit.size) else min(n, int(hit[0]) + 1 + extra)
    return O.Selection(blocks=np.sort(order[:k]), order=order, k_star=k, tau=float(m[order[k - 1]]),
                       c_prev=float(cs[k - 2]) if k > 1 else 0.0, c_star=float(cs[k - 1]),
                       all_blocks=k == n)


def _topk_generic(m, k_tokens, block, tie_desc=False, floor_blocks=False):
    m = np.asarray(m, np.float64)
    n = m.shape[0]
    ids = np.arange(n)
    order = np.lexsort(((-ids if tie_desc else ids), -m))
    kb = max(1, k_tokens // block) if floor_blocks else -(-k_tokens // block)
    k = min(kb, n)
    cs = np.cumsum(m[order])
    return O.Selection(blocks=np.sort(order[:k]), order=order, k_star=k, tau=float(m[order[k - 1]]),
                       c_prev=float(cs[k - 2]) if k > 1 else 0.0, c_star=float(cs[k - 1]),
                       all_blocks=k == n)


def _bf16_truncate(x):
    from fractions import Fraction
    v = float(Fraction(x))
    return int(np.float32(v).view(np.uint32) >> 16)


def _index_key_drops_last_dim(w_k_h, k_pre):
    from fractions import Fraction
    w = O.bf16_to_f64(w_k_h).reshape(16, 128)
    k = O.bf16_to_f64(k_pre).reshape(128)
    return np.array([O.bf16_round(sum((Fraction(float(w[i, d])) * Fraction(float(k[d])) for d in range(127)),
                                      Fraction(0))) for i in range(16)], dtype=np.uint16)


def _attend_no_scale(q, K, V, tokens):
    tokens = np.asarray(tokens, np.int64)
    if tokens.size == 0:
        return np.zeros(128), float("-inf")
    lg = O.bf16_to_f64(K[tokens]) @ O.bf16_to_f64(q)
    w = np.exp(lg - lg.max())
    return (w @ O.bf16_to_f64(V[tokens])) / w.sum(), float(lg.max() + np.log(w.sum()))


def _attend_lost_value(q, K, V, tokens):
    # the printed O_h(m) taken literally: no value vector
    tokens = np.asarray(tokens, np.int64)
    if tokens.size == 0:
        return np.zeros(128), float("-inf")
    lg = O.bf16_to_f64(K[tokens]) @ O.bf16_to_f64(q) / np.sqrt(128)
    w = np.exp(lg - lg.max())
    return np.full(128, (w / w.sum()).sum()), float(lg.max() + np.log(w.sum()))


def _local_off_by_one(n, window, sinks):
    return np.union1d(np.arange(min(sinks, n)), np.arange(max(0, n - window - 1), n)).astype(np.int64)


def _merge_unweighted(o_parts, lse_parts):
    lse = np.asarray(lse_parts, np.float64)
    live = np.isfinite(lse)
    return np.asarray(o_parts)[live].mean(axis=0), float(np.logaddexp.reduce(lse[live]))


def _retrieval_uses_wk(inp, b, r):
    saved = inp.w_q
    try:
        inp.w_q = inp.w_k
        return _orig["retrieval_head"](inp, b, r)
    finally:
        inp.w_q = saved


def _retrieval_wrong_group(inp, b, r):
    cfg = inp.cfg
    n = int(inp.seq_lens[b])
    hq = int(inp.ret_heads[r])
    kv = hq % cfg.Hkv
    qi = O.index_query(inp.w_q[r], inp.q_pre[b, hq])
    m = O.block_masses(O.index_scores(qi, inp.k_idx[b, r, :n]), cfg.block)
    sel = O.select_top_p(m, float(inp.top_p[b, r]))
    toks = O.block_tokens(sel.blocks, cfg.block, n)
    o, lse = O.attend(inp.q[b, hq], inp.k_cache[b, kv], inp.v_cache[b, kv], toks)
    return O.HeadResult(out=o, lse=lse, tokens=toks, masses=m, selection=sel)


def _prefill_excludes_self(i, retrieval, window, sinks):
    return _orig["prefill_tokens"](i - 1, retrieval, window, sinks) if i > 0 else np.zeros(1, np.int64)


def _prefill_sees_next(i, retrieval, window, sinks):
    return np.arange(i + 2, dtype=np.int64) if retrieval else _orig["prefill_tokens"](i, retrieval, window, sinks)


def _prefill_no_sinks(i, retrieval, window, sinks):
    return _orig["prefill_tokens"](i, retrieval, window, 0)


MUTANTS = [
    ("block_masses", _masses_per_block_softmax, [P.check_block_mass_worked, P.check_mass_vs_library]),
    ("block_masses", _masses_drop_partial, [P.check_block_mass_worked, P.check_mass_vs_library]),
    ("token_softmax", _softmax_wrong_sign, [P.check_block_mass_worked, P.check_mass_vs_library]),
    ("select_top_p", lambda m, p: _select_generic(m, p, tie_desc=True), [P.check_tie_break_worked]),
    ("select_top_p", lambda m, p: _select_generic(m, p, strict=True), [P.check_tie_break_worked]),
    ("select_top_p", lambda m, p: _select_generic(m, p, extra=1),
     [P.check_block_mass_worked, P.check_selection_bruteforce]),
    ("select_top_k", lambda m, k, b: _topk_generic(m, k, b, tie_desc=True), [P.check_topk_worked]),
    ("select_top_k", lambda m, k, b: _topk_generic(m, k, b, floor_blocks=True),
     [P.check_topk_worked, P.check_topk_bruteforce]),
    ("bf16_round", _bf16_truncate, [P.check_bf16_round]),
    ("index_key", _index_key_drops_last_dim, [P.check_index_key_vs_float64]),
    ("attend", _attend_no_scale, [P.check_attention_vs_sdpa]),
    ("attend", _attend_lost_value, [P.check_attention_vs_sdpa, P.check_attention_closed_forms]),
    ("local_tokens", _local_off_by_one, [P.check_local_tokens_worked]),
    ("merge_partials", _merge_unweighted, [P.check_merge_is_union]),
    ("retrieval_head", _retrieval_uses_wk, [P.check_dominant_needle]),
    ("retrieval_head", _retrieval_wrong_group, [P.check_gqa_mapping]),
    ("prefill_tokens", _prefill_excludes_self, [P.check_prefill_tokens_worked, P.check_prefill_one_hot_values]),
    ("prefill_tokens", _prefill_sees_next, [P.check_prefill_tokens_worked, P.check_prefill_vs_sdpa]),
    ("prefill_tokens", _prefill_no_sinks, [P.check_prefill_tokens_worked, P.check_prefill_vs_sdpa,
                                           P.check_prefill_one_hot_values]),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)),
                         ids=[f"{m[0]}:{m[1].__name__ if hasattr(m[1], '__name__') else i}"
                              for i, m in enumerate(MUTANTS)])
def test_mutant_is_caught(i, monkeypatch):
    name, fn, checks = MUTANTS[i]
    monkeypatch.setattr(O, name, fn)
    for chk in checks:
        with pytest.raises(AssertionError):
            chk()
