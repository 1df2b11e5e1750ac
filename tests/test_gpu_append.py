"""GPU parity of the decode-side cache append (rtp_cache_append): the token's K/V rows
and index keys are bit-exact against the oracle (index_key: exact sum, one rounding to
bf16), every other cache row is untouched, and a step after the append matches the
oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Run, check_outputs, check_selection, say
from long_context_sparse_amd import abi
from oracle import rtp_oracle as O

pytestmark = pytest.mark.gpu


def _bits(g, shape, scale=1.0):
    x = (g.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).cuda()


def _run_append(B, Hq, Hkv, n_ret, max_ctx, seq_lens, k_new, v_new, k_pre, w_k, ret_heads, caches):
    kc, vc, ki = (_dev(c) for c in caches)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    rh = torch.tensor(ret_heads, dtype=torch.int32, device="cuda")
    abi.rtp_cache_append(_dev(k_new), _dev(v_new), _dev(k_pre), _dev(w_k), sl, rh, B, Hq, Hkv, n_ret, max_ctx,
                         kc, vc, ki)
    torch.cuda.synchronize()
    return [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in (kc, vc, ki)]


def _expected(caches, seq_lens, k_new, v_new, k_pre, w_k, ret_heads, G):
    kc, vc, ki = (c.copy() for c in caches)
    for b, n in enumerate(seq_lens):
        kc[b, :, n - 1] = k_new[b]
        vc[b, :, n - 1] = v_new[b]
        for r, h in enumerate(ret_heads):
            ki[b, r, n - 1] = O.index_key(w_k[r], k_pre[b, h // G])
    return kc, vc, ki


@pytest.mark.parametrize("B,Hq,Hkv,n_ret,max_ctx,lens", [
    (3, 8, 2, 3, 300, (1, 150, 300)),      # first row, a middle row, the last row
    (2, 16, 2, 9, 64, (64, 7)),            # GQA 8, retrieval heads in both groups
    (1, 4, 4, 0, 32, (5,)),                # no retrieval heads: K/V rows only
])
def test_append_rows_bit_exact(B, Hq, Hkv, n_ret, max_ctx, lens):
    say(f"[gpu] append B={B} Hq={Hq} Hkv={Hkv} n_ret={n_ret} max_ctx={max_ctx} lens={lens}")
    g = np.random.default_rng(31)
    G = Hq // Hkv
    ret_heads = sorted(g.choice(Hq, size=n_ret, replace=False).tolist())
    caches = [_bits(g, (B, Hkv, max_ctx, 128)), _bits(g, (B, Hkv, max_ctx, 128)),
              _bits(g, (B, max(n_ret, 1), max_ctx, 16))]
    k_new, v_new, k_pre = _bits(g, (B, Hkv, 128)), _bits(g, (B, Hkv, 128)), _bits(g, (B, Hkv, 128))
    w_k = _bits(g, (max(n_ret, 1), 16, 128), 1 / np.sqrt(128))
    got = _run_append(B, Hq, Hkv, n_ret, max_ctx, lens, k_new, v_new, k_pre, w_k, ret_heads, caches)
    want = _expected(caches, lens, k_new, v_new, k_pre, w_k, ret_heads, G)
    for name, a, e in zip(("k_cache", "v_cache", "k_idx"), got, want):
        assert np.array_equal(a, e), name


def test_append_rounding_ties_and_ranges():
    """Keys that land exactly on bf16 ties (ties to even), bf16 subnormals and overflow
    to infinity, all in one append: each must match the oracle's single rounding."""
    B, Hq, Hkv, n_ret, max_ctx = 1, 4, 1, 4, 16
    f2b = lambda v: (np.float32(v).view(np.uint32) >> 16).astype(np.uint16)  # exact bf16 values only
    k_pre = np.zeros((B, Hkv, 128), np.uint16)
    k_pre[0, 0, 0] = f2b(1.0)
    k_pre[0, 0, 1] = f2b(1.0)
    w_k = np.zeros((n_ret, 16, 128), np.uint16)
    for i in range(16):
        w_k[0, i, 0], w_k[0, i, 1] = f2b(1.0), f2b((i + 1) * 2.0 ** -8)           # 1 + k 2^-8: ties
        w_k[1, i, 0], w_k[1, i, 1] = f2b(2.0 ** -127), f2b((i + 1) * 2.0 ** -133)  # subnormal sums
        w_k[2, i, 0], w_k[2, i, 1] = f2b(3.3e38), f2b(3.0e38 - i * 1e36)            # overflow
        w_k[3, i, 0], w_k[3, i, 1] = f2b(-(i + 1) * 0.1), f2b(0.1 * 2.0 ** -9)       # signed, inexact
    g = np.random.default_rng(32)
    caches = [_bits(g, (B, Hkv, max_ctx, 128)), _bits(g, (B, Hkv, max_ctx, 128)), _bits(g, (B, n_ret, max_ctx, 16))]
    k_new, v_new = _bits(g, (B, Hkv, 128)), _bits(g, (B, Hkv, 128))
    got = _run_append(B, Hq, Hkv, n_ret, max_ctx, (9,), k_new, v_new, k_pre, w_k, [0, 1, 2, 3], caches)
    want = _expected(caches, (9,), k_new, v_new, k_pre, w_k, [0, 1, 2, 3], 4)
    assert got[2][0, 0, 8].tolist() == [0x3F80 + j for j in [0, 1, 2, 2, 2, 3, 4, 4, 4, 5, 6, 6, 6, 7, 8, 8]]
    assert np.array_equal(got[2], want[2])
    assert (got[2][0, 2, 8] == 0x7F80).all()


@pytest.mark.parametrize("name", ["ctx32k", "ctx1m"])
def test_append_then_step(name):
    """At a bench workload's full size: the last token's rows are overwritten with junk,
    the append restores them from the token (its pre-RoPE key is its key: no RoPE in
    these inputs), the index keys equal the oracle's, and the step after it passes."""
    cfg = W.get_config(name)
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    B, G = cfg.B, cfg.Hq // cfg.Hkv
    lens = [int(n) for n in inp.seq_lens]
    k_new = np.stack([inp.k_cache[b, :, n - 1] for b, n in enumerate(lens)])
    v_new = np.stack([inp.v_cache[b, :, n - 1] for b, n in enumerate(lens)])
    for b, n in enumerate(lens):                       # junk in the rows the append must write
        t["k_cache"][b, :, n - 1] = 7.0
        t["v_cache"][b, :, n - 1] = -7.0
        t["k_idx"][b, :, n - 1] = 3.0
    abi.rtp_cache_append(_dev(k_new), _dev(v_new), _dev(k_new), _dev(inp.w_k) if cfg.n_ret else None,
                         t["seq_lens"], t["ret_heads"], B, cfg.Hq, cfg.Hkv, cfg.n_ret, cfg.max_ctx,
                         t["k_cache"], t["v_cache"], t["k_idx"])
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        kc = t["k_cache"][b, :, n - 1].view(torch.int16).cpu().numpy().view(np.uint16)
        vc = t["v_cache"][b, :, n - 1].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(kc, k_new[b]) and np.array_equal(vc, v_new[b])
        ki = t["k_idx"][b, :, n - 1].view(torch.int16).cpu().numpy().view(np.uint16)
        for r, h in enumerate(inp.ret_heads):
            assert np.array_equal(ki[r], O.index_key(inp.w_k[r], k_new[b, int(h) // G])), (b, r)
            inp.k_idx[b, r, n - 1] = ki[r]           # the oracle sees the appended keys
    run = Run(inp, tensors=t, tag=f"{name} after append")
    check_selection(run)
    check_outputs(run, [(b, int(h)) for b in range(B) for h in inp.ret_heads])


def _boundary_vectors():
    """w and k bit vectors whose exact dot products sit on or next to a bf16 rounding
    boundary (ties with tails of either sign far below fp64's reach, cancellation,
    subnormal and overflowing sums, signed zeros), plus ties with random tails."""
    from key_cases import CASES, vec
    ws = [CASES[n][0] for n in sorted(CASES)]
    ks = [CASES[n][1] for n in sorted(CASES)]
    g = np.random.default_rng(77)
    for it in range(19):
        n = int(g.integers(-20, 20))
        e = n - 1 - int(g.integers(20, 90))
        sgn = 1.0 if it % 2 else -1.0
        w, k = vec((float(int(g.integers(128, 256))) * 2.0 ** n, 1.0), (2.0 ** (n - 1), 1.0),
                   (sgn * 2.0 ** (e // 2), 2.0 ** (e - e // 2)))
        ws.append(w)
        ks.append(k)
    return np.stack(ws), np.stack(ks)


def test_append_keys_exact_sum_rounded_once():
    """rtp_cache_append's index keys against oracle.index_key (the exact sum rounded once)
    on every pairing of 32 boundary w rows (two retrieval heads of 16 dims) with 32
    boundary k vectors (one per sequence): among them the tie-with-tail input that a
    rounded fp64 sum gets wrong, its negative and its just-below-tie twin."""
    ws, ks = _boundary_vectors()
    n_ret, B = 2, ks.shape[0]
    say(f"[gpu] append keys: {B} k vectors x {ws.shape[0]} w rows")
    w_k = ws.reshape(n_ret, 16, 128)
    Hq = Hkv = n_ret  # one KV group per retrieval head; every group sees the same k_pre
    k_pre = np.repeat(ks[:, None, :], Hkv, axis=1)
    g = np.random.default_rng(3)
    max_ctx = 4
    lens = [1 + (b % max_ctx) for b in range(B)]
    caches = [_bits(g, (B, Hkv, max_ctx, 128)), _bits(g, (B, Hkv, max_ctx, 128)), _bits(g, (B, n_ret, max_ctx, 16))]
    k_new, v_new = _bits(g, (B, Hkv, 128)), _bits(g, (B, Hkv, 128))
    got = _run_append(B, Hq, Hkv, n_ret, max_ctx, lens, k_new, v_new, k_pre, w_k, list(range(n_ret)), caches)
    ki = got[2]
    bad = []
    for b in range(B):
        for r in range(n_ret):
            want = O.index_key(w_k[r], ks[b])
            have = ki[b, r, lens[b] - 1]
            if not np.array_equal(have, want):
                bad.append((b, r, [hex(x) for x in have[have != want]], [hex(x) for x in want[have != want]]))
    assert not bad, bad[:4]
    # the counterexample pairing itself: w row "tie_plus_tail" with its own k
    from key_cases import CASES
    i = sorted(CASES).index("tie_plus_tail")
    assert ki[i, i // 16, lens[i] - 1, i % 16] == 0x3F81


def test_prompt_keys_exact_sum_rounded_once():
    """rtp_prefill_index_keys on the same boundary pairings: 32 prompt rows (the k
    vectors) against 32 w rows, bit for bit against oracle.index_key."""
    ws, ks = _boundary_vectors()
    n_ret, T = 2, ks.shape[0]
    say(f"[gpu] prompt keys: {T} rows x {ws.shape[0]} w rows")
    w_k = ws.reshape(n_ret, 16, 128)
    Hq, Hkv = 4, 2
    k_pre = np.repeat(ks[None, None], Hkv, axis=1)          # [1, Hkv, T, 128]
    ret = [1, 2]                                             # KV groups 0 and 1
    k_idx = torch.zeros((1, n_ret, T, 16), dtype=torch.int16, device="cuda")
    sl = torch.tensor([T], dtype=torch.int32, device="cuda")
    rh = torch.tensor(ret, dtype=torch.int32, device="cuda")
    abi.rtp_prefill_index_keys(_dev(k_pre), _dev(w_k), sl, rh, 1, Hq, Hkv, n_ret, T, k_idx)
    torch.cuda.synchronize()
    ki = k_idx.cpu().numpy().view(np.uint16)
    bad = []
    for t in range(T):
        for r in range(n_ret):
            want = O.index_key(w_k[r], ks[t])
            if not np.array_equal(ki[0, r, t], want):
                bad.append((t, r))
    assert not bad, bad[:8]
