"""Pins for the fp64 oracle against facts fixed outside it.

Each ``check_*`` helper raises AssertionError on a mismatch; the tests call them
as they are, and tests/test_oracle_mutations.py calls them against oracles with
planted mistakes to show that each mistake is caught.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import workloads as W
from oracle import rtp_oracle as O
from oracle import accept as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


# ------------------------------------------------------------------ index (a1-a3)
def check_index_worked():
    g = _gold("index_worked.json")
    Wq = np.zeros((16, 128), np.float32)
    for i in range(16):
        Wq[i, 8 * i] = 1.0
    q = np.array([(k % 7) - 3 for k in range(128)], np.float32)
    qi = O.index_query(_bits(Wq), _bits(q))
    assert np.array_equal(qi, np.array(g["q_idx"], np.float64))
    n = g["n_tokens"]
    K = np.zeros((n, 16), np.float32)
    K[np.arange(n), np.arange(n) % 16] = 1.0
    s = O.index_scores(qi, _bits(K))
    assert np.array_equal(s, np.array([g["q_idx"][t % 16] for t in range(n)], np.float64))


def check_block_mass_worked():
    g = _gold("block_mass_worked.json")
    s = np.log(np.array(g["scores_ln_of"], np.float64))
    m = O.block_masses(s, g["block"])
    want = np.array(g["mass_numerators"], np.float64) / g["mass_denominator"]
    assert m.shape == want.shape
    assert np.allclose(m, want, rtol=0, atol=1e-15)
    for c in g["selections"]:
        sel = O.select_top_p(m, c["p"])
        assert sel.blocks.tolist() == c["blocks"], (c, sel.blocks)
        assert abs(sel.tau - c["tau_num"] / g["mass_denominator"]) < 1e-15


def check_tie_break_worked():
    g = _gold("tie_break_worked.json")
    for case in g["cases"]:
        s = np.log(np.array(case["scores_ln_of"], np.float64))
        m = O.block_masses(s, case["block"])
        want = np.array(case["mass_numerators"], np.float64) / case["mass_denominator"]
        assert np.allclose(m, want, rtol=0, atol=1e-15)
        for c in case["selections"]:
            assert O.select_top_p(m, c["p"]).blocks.tolist() == c["blocks"], c


def check_mass_vs_library():
    g = np.random.default_rng(5)
    for n, bk in ((1, 64), (63, 64), (64, 64), (1000, 64), (777, 128)):
        s = g.standard_normal(n) * 4.0
        m = O.block_masses(s, bk)
        assert m.shape[0] == -(-n // bk)
        assert abs(m.sum() - 1.0) < 1e-12
        lse = scipy.special.logsumexp(s)
        for j in range(m.shape[0]):
            blk = s[j * bk:(j + 1) * bk]
            assert abs(m[j] - math.exp(scipy.special.logsumexp(blk) - lse)) < 1e-12
        ref = torch.softmax(torch.from_numpy(s), dim=0).numpy()
        assert np.allclose(O.token_softmax(s), ref, rtol=0, atol=1e-15)


# ------------------------------------------------------------- selection (a4-a5)
def _greedy_python(m, p):
    """Independent greedy: pure-Python sort and running sum."""
    order = sorted(range(len(m)), key=lambda j: (-m[j], j))
    if p >= 1.0:
        return sorted(order)
    tot = 0.0
    out = []
    for j in order:
        out.append(j)
        tot += m[j]
        if tot >= p:
            break
    return sorted(out)


def check_selection_bruteforce(trials=300, seed=7):
    g = np.random.default_rng(seed)
    for t in range(trials):
        n = int(g.integers(1, 13))
        if t % 3 == 0:
            m = g.dirichlet(np.ones(n) * 0.3)
        elif t % 3 == 1:
            m = g.integers(1, 4, size=n).astype(np.float64)   # many exact ties
            m /= m.sum()
        else:
            m = g.dirichlet(np.ones(n) * 3.0)
        p = float(g.choice([0.3, 0.5, 0.8, 0.9, 0.95, 0.99, float(g.uniform(0.05, 0.999))]))
        # keep p off exact subset sums (those crossings are pinned by the golden tie cases)
        p += 3.3e-7
        sel = O.select_top_p(m, p)
        assert sel.blocks.tolist() == _greedy_python(m.tolist(), p)
        # exhaustive: the oracle set has the fewest blocks among all subsets reaching p,
        # and the largest mass among subsets of that size
        best_k, best_mass = None, -1.0
        for k in range(1, n + 1):
            for sub in itertools.combinations(range(n), k):
                ms = sum(m[list(sub)])
                if ms >= p - 1e-12:
                    best_mass = max(best_mass, ms)
            if best_mass >= 0:
                best_k = k
                break
        assert sel.k_star == best_k, (m, p, sel.k_star, best_k)
        assert abs(m[sel.blocks].sum() - best_mass) < 1e-12
        # coverage and minimality invariants
        tot = m[sel.blocks].sum()
        assert tot >= p - 1e-12
        assert tot - m[sel.blocks].min() < p


def check_p_one_selects_all():
    g = np.random.default_rng(8)
    m = g.dirichlet(np.ones(50))
    m[3] = 0.0
    assert O.select_top_p(m, 1.0).blocks.tolist() == list(range(50))


def check_dominant_needle():
    cfg = W.custom_config(B=1, Hkv=1, Hq=4, n_ret=2, ctx=(2048,), kind="depth_needles",
                          top_p=(0.9, 0.95))
    inp = W.make_inputs(cfg)
    for r in range(2):
        res = O.retrieval_head(inp, 0, r)
        need = inp.needles[(0, r)]
        # one dominant needle block per depth; three depths -> three equal blocks
        assert res.selection.blocks.tolist() == sorted(need)
    cfg1 = W.custom_config(B=2, Hkv=2, Hq=4, n_ret=2, ctx=(3000, 1500), kind="peaked_diffuse",
                           top_p=(0.95, 0.95))
    inp1 = W.make_inputs(cfg1)
    for (b, r), pk in inp1.peaked.items():
        if pk:
            res = O.retrieval_head(inp1, b, r)
            assert res.selection.blocks.tolist() == inp1.needles[(b, r)]
            assert res.masses[inp1.needles[(b, r)][0]] > 0.95


# ------------------------------------------------------- static top-k (next row f1)
def check_topk_worked():
    """Hand-worked: masses [0.1, 0.4, 0.4, 0.1] at block 64; the budget is counted in
    tokens and rounded up to whole blocks; ties go to the lower block id."""
    m = np.array([0.1, 0.4, 0.4, 0.1])
    assert O.select_top_k(m, 64, 64).blocks.tolist() == [1]           # 1 block: tie 1/2 -> 1
    assert O.select_top_k(m, 65, 64).blocks.tolist() == [1, 2]        # 2 blocks
    assert O.select_top_k(m, 129, 64).blocks.tolist() == [0, 1, 2]   # 3 blocks: tie 0/3 -> 0
    assert O.select_top_k(m, 10000, 64).blocks.tolist() == [0, 1, 2, 3]
    assert O.select_top_k(m, 10000, 64).all_blocks
    assert O.select_top_k(m, 128, 128).blocks.tolist() == [1]         # block 128: 1 block
    assert O.select_top_k(m, 4096, 64).k_star == 4


def check_topk_bruteforce(trials=300, seed=11):
    """Against exhaustive search on tiny inputs: the kept set is a subset of the budget's
    size with the largest mass, and among those the one a pure-Python sort by (mass
    descending, id ascending) picks."""
    g = np.random.default_rng(seed)
    for t in range(trials):
        n = int(g.integers(1, 11))
        m = g.dirichlet(np.ones(n) * 0.5) if t % 2 else g.integers(1, 4, size=n) / 10.0
        block = int(g.choice([64, 128]))
        k_tokens = int(g.integers(1, (n + 2) * block))
        kb = -(-k_tokens // block)
        sel = O.select_top_k(m, k_tokens, block)
        k = min(kb, n)
        want = sorted(sorted(range(n), key=lambda j: (-m[j], j))[:k])
        assert sel.blocks.tolist() == want, (m, k_tokens, block)
        best = max(sum(m[list(sub)]) for sub in itertools.combinations(range(n), k))
        assert abs(m[sel.blocks].sum() - best) < 1e-12


def check_topk_matches_topp_prefix(trials=200, seed=12):
    """Both rules take a prefix of the same order: a budget of exactly the top-p set's
    size (in tokens) keeps the top-p set."""
    g = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(g.integers(1, 200))
        m = g.dirichlet(np.ones(n) * float(g.choice([0.05, 0.5, 5.0])))
        p = float(g.uniform(0.1, 0.999))
        sp = O.select_top_p(m, p)
        block = 64
        sk = O.select_top_k(m, sp.k_star * block - int(g.integers(0, block)), block)
        assert sk.blocks.tolist() == sp.blocks.tolist()


# ---------------------------------------------------- cache append (next row f2)
def check_bf16_round():
    """Against torch's float32 -> bfloat16 conversion (nearest-even) on float32 values,
    and hand cases: ties to even, the subnormal range, overflow, signed zero."""
    x = np.random.default_rng(21).standard_normal(5000).astype(np.float32) * np.float32(7.0)
    x = np.concatenate([x, np.float32([1e-39, -3e-40, 1e-45, 3.3e38, -3.38e38, 1.17549435e-38])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([O.bf16_round(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert O.bf16_round(1.0 + 2.0 ** -8) == 0x3F80          # tie -> even mantissa 0
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even mantissa 2
    assert O.bf16_round(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81   # above the tie
    assert O.bf16_round(2.0 ** -130) == 0x0008              # subnormal: 8 quanta of 2^-133
    assert O.bf16_round(2.0 ** -126 * (1 - 2.0 ** -20)) == 0x0080   # rounds up to the smallest normal
    assert O.bf16_round(3.5e38) == 0x7F80 and O.bf16_round(-0.0) == 0x8000
    # a tie carried only by a term far below float64 precision of the sum: exact input
    from fractions import Fraction
    assert O.bf16_round(Fraction(1) + Fraction(1, 256) + Fraction(1, 2 ** 90)) == 0x3F81


def check_index_key_worked():
    """Hand-worked: k_pre = (1, 1, 0, ...); row i of W^K = (1, (i + 1) 2^-8, 0, ...), so
    key i = 1 + (i + 1) 2^-8, which bf16 (spacing 2^-7 at 1) rounds to 1 + 2 j 2^-8
    with j the even neighbour at the odd (tied) values."""
    def bits(v):
        return np.float32(v).view(np.uint32) >> 16
    k = np.zeros(128, np.uint16)
    k[0] = k[1] = bits(1.0)
    w = np.zeros((16, 128), np.uint16)
    for i in range(16):
        w[i, 0] = bits(1.0)
        w[i, 1] = bits((i + 1) * 2.0 ** -8)
    j = [0, 1, 2, 2, 2, 3, 4, 4, 4, 5, 6, 6, 6, 7, 8, 8]
    assert O.index_key(w, k).tolist() == [0x3F80 + v for v in j]
    # sign and scale: negating k negates every key; scaling k by 2 adds one to each exponent
    assert (O.index_key(w, k ^ np.uint16(0x8000) * (k != 0)) == (O.index_key(w, k) | 0x8000)).all()
    k2 = k.copy()
    k2[:2] = bits(2.0)
    assert (O.index_key(w, k2) == O.index_key(w, k) + 0x80).all()


def check_index_key_vs_float64():
    """On random bf16 inputs whose products span well under 53 bits, the exact sum equals
    the float64 sum, so the key equals torch's rounding of the float64 matvec (through
    float32 only where that cannot double-round: checked against the exact rounding)."""
    g = np.random.default_rng(22)
    w = (np.float32(g.standard_normal((16, 128)) / np.sqrt(128)).view(np.uint32) >> 16).astype(np.uint16)
    k = (np.float32(g.standard_normal(128)).view(np.uint32) >> 16).astype(np.uint16)
    wf = O.bf16_to_f64(w)
    kf = O.bf16_to_f64(k)
    ref = [O.bf16_round(float(np.dot(wf[i], kf))) for i in range(16)]
    assert O.index_key(w, k).tolist() == ref


# ------------------------------------------------------------ attention (a6-a8)
def _sdpa(q, K, V):
    qt = torch.from_numpy(O.bf16_to_f64(q))[None, None, None, :]
    kt = torch.from_numpy(O.bf16_to_f64(K))[None, None]
    vt = torch.from_numpy(O.bf16_to_f64(V))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0, 0].numpy()


def check_attention_vs_sdpa():
    g = np.random.default_rng(9)
    for n in (1, 5, 64, 300):
        q = _bits(g.standard_normal(128))
        K = _bits(g.standard_normal((n, 128)) * 1.5)
        V = _bits(g.standard_normal((n, 128)))
        o, lse = O.attend(q, K, V, np.arange(n))
        assert np.allclose(o, _sdpa(q, K, V), rtol=0, atol=1e-12)
        logits = O.bf16_to_f64(K) @ O.bf16_to_f64(q) / math.sqrt(128)
        assert abs(lse - scipy.special.logsumexp(logits)) < 1e-11
        sub = np.array(sorted(g.choice(n, size=max(1, n // 2), replace=False)))
        o2, _ = O.attend(q, K, V, sub)
        assert np.allclose(o2, _sdpa(q, K[sub], V[sub]), rtol=0, atol=1e-12)


def check_attention_closed_forms():
    g = np.random.default_rng(10)
    V = _bits(g.standard_normal((6, 128)))
    q = _bits(g.standard_normal(128))
    K = _bits(g.standard_normal((6, 128)))
    o, _ = O.attend(q, K, V, np.array([4]))
    assert np.array_equal(o, O.bf16_to_f64(V[4]))            # single token -> its value
    Ks = np.tile(K[2], (6, 1))
    o, lse = O.attend(q, Ks, V, np.arange(6))
    assert np.allclose(o, O.bf16_to_f64(V).mean(axis=0), rtol=0, atol=1e-15)   # equal keys -> mean
    # a key 64 * 64 / sqrt(128) below the others carries no weight: uniform over the rest
    q1 = np.zeros(128, np.float32); q1[0] = 64.0
    K1 = np.zeros((3, 128), np.float32); K1[2, 0] = -64.0
    o, lse = O.attend(_bits(q1), _bits(K1), V[:3], np.arange(3))
    assert np.allclose(o, (O.bf16_to_f64(V[0]) + O.bf16_to_f64(V[1])) / 2, rtol=0, atol=1e-15)
    assert abs(lse - math.log(2.0)) < 1e-15
    o, lse = O.attend(q, K, V, np.array([], np.int64))
    assert lse == float("-inf") and not o.any()


def check_merge_is_union():
    g = np.random.default_rng(11)
    n = 500
    q = _bits(g.standard_normal(128))
    K = _bits(g.standard_normal((n, 128)))
    V = _bits(g.standard_normal((n, 128)))
    full, lse_full = O.attend(q, K, V, np.arange(n))
    cuts = [0, 17, 17, 200, 333, n]            # includes an empty part
    parts = [O.attend(q, K, V, np.arange(a, b)) for a, b in zip(cuts[:-1], cuts[1:])]
    o, L = O.merge_partials(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
    assert np.allclose(o, full, rtol=0, atol=1e-13)
    assert abs(L - lse_full) < 1e-12


def check_local_tokens_worked():
    g = _gold("local_window_worked.json")
    for c in g["cases"]:
        t = O.local_tokens(c["N"], c["W"], c["S"])
        if "tokens" in c:
            assert t.tolist() == c["tokens"], c
        else:
            assert t.size == c["tokens_count"] and t[:5].tolist() == c["first"] and t[-1] == c["last"]
    rng = np.random.default_rng(12)
    for _ in range(200):       # brute-force predicate
        n = int(rng.integers(1, 40)); w = int(rng.integers(0, 45)); s = int(rng.integers(0, 8))
        want = [t for t in range(n) if t < s or t >= n - w]
        assert O.local_tokens(n, w, s).tolist() == want


def check_local_reduces_to_dense():
    cfg = W.custom_config(B=1, Hkv=1, Hq=4, n_ret=1, ctx=(300,), window=296, sinks=4)
    inp = W.make_inputs(cfg)
    h = int(inp.loc_heads[0])
    assert np.array_equal(O.local_head(inp, 0, h).out, O.dense_head(inp, 0, h).out)
    cfg2 = W.custom_config(B=1, Hkv=1, Hq=4, n_ret=1, ctx=(300,), window=1, sinks=0)
    inp2 = W.make_inputs(cfg2)
    h = int(inp2.loc_heads[0])
    assert np.array_equal(O.local_head(inp2, 0, h).out, O.bf16_to_f64(inp2.v_cache[0, 0, 299]))


def check_p_one_is_dense():
    cfg = W.custom_config(B=1, Hkv=2, Hq=4, n_ret=2, ctx=(1500,), top_p=(1.0, 1.0), kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    for r in range(2):
        res = O.retrieval_head(inp, 0, r)
        dn = O.dense_head(inp, 0, int(inp.ret_heads[r]))
        assert np.array_equal(res.out, dn.out)
        kv = int(inp.ret_heads[r]) // 2
        assert np.allclose(dn.out, _sdpa(inp.q[0, inp.ret_heads[r]], inp.k_cache[0, kv, :1500],
                                         inp.v_cache[0, kv, :1500]), rtol=0, atol=1e-12)


def check_gqa_mapping():
    # retrieval head uses its own index cache and its KV group's K/V
    cfg = W.custom_config(B=1, Hkv=2, Hq=8, n_ret=2, ctx=(256,), ret_heads=(1, 6), top_p=(1.0, 1.0))
    inp = W.make_inputs(cfg)
    res = O.retrieval_head(inp, 0, 1)
    assert np.allclose(res.out, _sdpa(inp.q[0, 6], inp.k_cache[0, 1, :256], inp.v_cache[0, 1, :256]),
                       rtol=0, atol=1e-12)


# --------------------------------------------------------------------- prefill
def check_prefill_tokens_worked():
    # worked by hand from the rule (Review, Adaptive sparse attention: window + sink in
    # prefill for local heads, dense for retrieval heads; causal): W = 3, S = 2
    want = {0: [0], 1: [0, 1], 2: [0, 1, 2], 3: [0, 1, 2, 3], 4: [0, 1, 2, 3, 4], 5: [0, 1, 3, 4, 5],
            9: [0, 1, 7, 8, 9]}
    for i, t in want.items():
        assert O.prefill_tokens(i, False, 3, 2).tolist() == t, i
        assert O.prefill_tokens(i, True, 3, 2).tolist() == list(range(i + 1)), i
    assert O.prefill_tokens(5, False, 0, 2).tolist() == [0, 1]        # sinks only
    assert O.prefill_tokens(5, False, 1, 0).tolist() == [5]           # the token itself
    assert O.prefill_tokens(1, False, 0, 4).tolist() == [0, 1]        # sinks beyond the prompt so far


def _prefill_pin_inputs(N, Hq, Hkv, ret_heads, window, sinks, seed):
    # a second, longer prompt gives the first one rows past its end (a rule that looks
    # past position i then reads them instead of failing on an index)
    cfg = W.custom_config(B=2, Hkv=Hkv, Hq=Hq, n_ret=len(ret_heads), ret_heads=tuple(ret_heads), ctx=(N, N + 5),
                          window=window, sinks=sinks, seed=seed)
    return W.make_prefill_inputs(cfg)


def check_prefill_vs_sdpa():
    """Every row of every head against torch's attention in float64 with the causal /
    window + sink mask written as an elementwise predicate on (query i, key j)."""
    pin = _prefill_pin_inputs(70, 4, 2, (1,), 9, 3, 21)
    N, S, Wn = 70, 3, 9
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    for h in range(4):
        kv = h // 2
        qt = torch.from_numpy(O.bf16_to_f64(pin.q[0, h, :N]))[None, None]
        kt = torch.from_numpy(O.bf16_to_f64(pin.k[0, kv, :N]))[None, None]
        vt = torch.from_numpy(O.bf16_to_f64(pin.v[0, kv, :N]))[None, None]
        if h == 1:
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        else:
            m = torch.from_numpy((j <= i) & ((j < S) | (i - j < Wn)))
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
        assert np.allclose(O.prefill_head(pin, 0, h), ref[0, 0].numpy(), rtol=0, atol=1e-12), h


def check_prefill_one_hot_values():
    """Equal keys give uniform weights; V row j = e_j then shows each row's token set
    and weights directly: output[i, j] = 1 / |T_i| for j in T_i, else 0."""
    pin = _prefill_pin_inputs(100, 2, 1, (0,), 7, 2, 22)
    pin.k[0, 0, :100] = pin.k[0, 0, 0]
    one = W.f32_to_bf16_bits(np.float32([1.0]))[0]
    pin.v[0, 0, :100] = 0
    pin.v[0, 0, np.arange(100), np.arange(100)] = one
    for h, pred in ((0, lambda i, j: j <= i), (1, lambda i, j: j <= i and (j < 2 or j > i - 7))):
        out = O.prefill_head(pin, 0, h)
        for i in range(100):
            T = [j for j in range(100) if pred(i, j)]
            want = np.zeros(128)
            want[T] = 1.0 / len(T)
            assert np.allclose(out[i], want, rtol=0, atol=1e-15), (h, i)


# ------------------------------------------------------------------ acceptance
def check_acceptance_rule():
    m = np.array([0.3, 0.3, 0.2, 0.1, 0.1])
    sel = O.select_top_p(m, 0.75)              # 0.3, 0.3, 0.2 -> {0, 1, 2}
    assert A.accept_selection(m, 0.75, [0, 1, 2], sel)[0]
    assert not A.accept_selection(m, 0.75, [0, 1], sel)[0]          # R1/R3
    assert not A.accept_selection(m, 0.75, [0, 1, 2, 3], sel)[0]    # R2/R4
    # equal needles: dropping one violates R3 even though its mass equals tau
    m2 = np.array([0.49, 0.49, 0.02])
    assert A.accept_selection(m2, 0.9, [0, 1])[0]
    assert not A.accept_selection(m2, 0.9, [0, 2])[0]
    # ambiguous crossing within eps: one more block is acceptable
    m3 = np.array([0.5, 0.4000000001, 0.0999999999])
    assert A.accept_selection(m3, 0.9, [0, 1])[0]
    assert A.accept_selection(m3, 0.9, [0, 1, 2])[0]
    assert A.accept_selection(m, 1.0, [0, 1, 2, 3, 4])[0]
    assert not A.accept_selection(m, 1.0, [0, 1, 2, 3])[0]
    # static top-k: exact size, no lower block in place of a higher one; ties either way
    mk = np.array([0.1, 0.4, 0.4, 0.1])
    assert A.accept_topk(mk, 65, 64, [1, 2])[0]
    assert not A.accept_topk(mk, 65, 64, [1])[0]                 # too few
    assert not A.accept_topk(mk, 65, 64, [0, 1, 2])[0]           # too many
    assert not A.accept_topk(mk, 65, 64, [0, 1])[0]              # 0.1 in place of 0.4
    assert A.accept_topk(mk, 64, 64, [2])[0]                     # tie at the threshold
    assert A.accept_topk(mk, 129, 64, [1, 2, 3])[0]
    assert A.accept_topk(mk, 9999, 64, [0, 1, 2, 3])[0]


CHECKS = [check_index_worked, check_block_mass_worked, check_tie_break_worked, check_mass_vs_library,
          check_selection_bruteforce, check_p_one_selects_all, check_dominant_needle,
          check_topk_worked, check_topk_bruteforce, check_topk_matches_topp_prefix,
          check_bf16_round, check_index_key_worked, check_index_key_vs_float64,
          check_attention_vs_sdpa, check_attention_closed_forms, check_merge_is_union,
          check_local_tokens_worked, check_local_reduces_to_dense, check_p_one_is_dense,
          check_gqa_mapping, check_acceptance_rule,
          check_prefill_tokens_worked, check_prefill_vs_sdpa, check_prefill_one_hot_values]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check()
