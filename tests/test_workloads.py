"""The seeded input generator: determinism, bf16 rounding, planting."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rne_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.005859375, 3.0e-20, 7e30], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_direct_rounding():
    g = np.random.default_rng(1)
    x = g.standard_normal(100000) * 10.0
    bits = W.f64_to_bf16_bits(x)
    y = W.bf16_bits_to_f32(bits).astype(np.float64)
    # nearest: the error is at most half a bf16 ulp of x
    ulp = 2.0 ** (np.floor(np.log2(np.abs(x))) - 7)
    assert np.all(np.abs(y - x) <= 0.5 * ulp + 1e-300)
    # exact ties go to even
    t = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])
    assert W.bf16_bits_to_f32(W.f64_to_bf16_bits(t)).tolist() == [1.0, 1.0 + 2.0 ** -6]


def test_determinism_and_seed_sensitivity():
    cfg = W.custom_config(B=2, Hkv=2, Hq=8, n_ret=3, ctx=(700, 333), kind="peaked_diffuse")
    a = W.make_inputs(cfg)
    b = W.make_inputs(cfg, workers=1)
    for f in ("q", "w_q", "w_k", "k_cache", "v_cache", "k_idx", "ret_heads", "top_p"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = W.make_inputs(cfg, seed=cfg.seed + 1)
    assert not np.array_equal(a.k_cache, c.k_cache)


def test_padding_and_poison():
    cfg = W.custom_config(B=2, ctx=(100, 37), kind="random")
    inp = W.make_inputs(cfg, pad_value=int(W.BF16_NAN))
    assert np.all(inp.k_cache[1, :, 37:] == W.BF16_NAN)
    assert np.all(inp.k_idx[1, :, 37:] == W.BF16_NAN)
    assert not np.any(inp.k_cache[1, :, :37] == W.BF16_NAN)


def test_named_configs_shapes():
    c = W.CONFIGS
    assert (c["tiny"].B, c["tiny"].Hq, c["tiny"].n_ret, c["tiny"].max_ctx, c["tiny"].block) == (1, 4, 4, 4096, 64)
    assert (c["ctx32k"].Hkv, c["ctx32k"].Hq, c["ctx32k"].n_ret, c["ctx32k"].window) == (8, 32, 8, 1024)
    assert (c["ctx128k"].B, c["ctx128k"].max_ctx) == (4, 131072)
    assert (c["ctx1m"].max_ctx, c["ctx1m"].block, c["ctx1m"].split_tokens) == (1 << 20, 128, 65536)
    m = c["mixed"]
    assert m.B == 16 and all(8192 <= n <= 262144 for n in m.ctx) and m.n_ret == 6
    assert set(m.top_p) <= {0.9, 0.95, 0.99}


def _score(inp, b, r, toks):
    qi = W.bf16_bits_to_f32(inp.w_q[r]).astype(np.float64) @ W.bf16_bits_to_f32(inp.q[b, inp.ret_heads[r]]).astype(np.float64)
    return W.bf16_bits_to_f32(inp.k_idx[b, r, toks]).astype(np.float64) @ qi


def test_peaked_margin_survives_bf16():
    cfg = W.custom_config(B=2, Hkv=2, Hq=8, n_ret=4, ctx=(3000, 2500), kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    npk = 0
    for (b, r), pk in inp.peaked.items():
        if not pk:
            continue
        npk += 1
        n = int(inp.seq_lens[b])
        (j,) = inp.needles[(b, r)]
        toks = np.arange(n)
        s = _score(inp, b, r, toks)
        inn = (toks // cfg.block) == j
        assert s[inn].min() - s[~inn].max() > 5.9
    assert npk == 4


def test_tiny_needles_planted():
    inp = W.make_inputs(W.get_config("tiny"))
    blocks = inp.needles[(0, 0)]
    assert len(blocks) == 2
    for r in range(4):
        assert inp.needles[(0, r)] == blocks
        s = _score(inp, 0, r, np.arange(4096))
        nb = np.zeros(4096, bool)
        for j in blocks:
            nb[j * 64:(j + 1) * 64] = True
        assert s[nb].min() > s[~nb].max() + 10
