"""GPU parity of the prefill calls against the oracle: rtp_prefill_attn (causal; local
heads window + sink, retrieval heads dense) on every row of small prompts that span
several tiles with ragged ends, and on sampled rows of a 32K prompt; and
rtp_prefill_index_keys bit-exact.  Rows past each prompt are poisoned with NaN and must
be neither read nor written."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say
from long_context_sparse_amd import abi
from oracle import accept as A
from oracle import rtp_oracle as O

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _run(pin):
    cfg = pin.cfg
    t = W.prefill_to_device(pin)
    out = torch.full((cfg.B, cfg.Hq, cfg.max_ctx, 128), SENTINEL, dtype=torch.float32, device="cuda")
    abi.rtp_prefill_attn(t["q"], t["k"], t["v"], t["seq_lens"], t["ret_heads"], cfg.B, cfg.Hq, cfg.Hkv, cfg.n_ret,
                         cfg.max_ctx, cfg.window, cfg.sinks, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), t


def _check_rows(pin, out, items):
    """items: (b, h, rows); compares with the oracle and checks rows past the prompt."""
    g, o = [], []
    for b, h, rows in items:
        g.append(out[b, h, rows].astype(np.float64))
        o.append(O.prefill_head(pin, b, h, rows))
    g, o = np.concatenate(g), np.concatenate(o)
    ok, ma, mr = A.outputs_ok(g, o)
    say(f"      prefill outputs: {g.shape[0]} rows, max-abs {ma:.3e}, mean-rel {mr:.3e}")
    assert ok, f"prefill outputs out of tolerance: max-abs {ma:.3e} mean-rel {mr:.3e}"
    for b, n in enumerate(pin.seq_lens):
        assert (out[b, :, int(n):] == SENTINEL).all(), f"rows past the prompt written (b={b})"


SMALL = {
    # name: (B, Hq, Hkv, ret_heads, ctx, window, sinks)
    "mixed_gqa4": (2, 8, 2, (0, 5), (700, 333), 100, 4),
    "gqa1_window_only": (1, 3, 3, (1,), (1000,), 64, 0),
    "gqa8_sinks_only": (2, 8, 1, (7,), (257, 129), 0, 70),
    "window_covers_prompt": (1, 4, 2, (), (300,), 512, 4),
    "window_one": (1, 2, 1, (), (200,), 1, 0),
    "all_retrieval": (2, 4, 4, (0, 1, 2, 3), (128, 1), 16, 4),
    "tiny_prompts": (4, 4, 1, (2,), (1, 2, 63, 65), 7, 2),
    "long_window_edge": (1, 4, 1, (3,), (2100,), 1000, 4),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_small_all_rows(name):
    B, Hq, Hkv, ret, ctx, win, sinks = SMALL[name]
    cfg = W.custom_config(name=f"prefill_{name}", seed=60 + len(name), B=B, Hq=Hq, Hkv=Hkv, n_ret=len(ret),
                          ret_heads=ret, ctx=ctx, window=win, sinks=sinks)
    pin = W.make_prefill_inputs(cfg, pad_value=W.BF16_NAN)
    say(f"[gpu] prefill {name}: B={B} Hq={Hq} Hkv={Hkv} ret={ret} ctx={ctx} window={win} sinks={sinks}")
    out, _ = _run(pin)
    items = [(b, h, list(range(int(n)))) for b, n in enumerate(pin.seq_lens) for h in range(Hq)]
    _check_rows(pin, out, items)


BENCH_RET = (3, 9, 15, 20, 30)  # the benchmark's prefill configuration: 32 query / 8 KV heads


def _bench_rows(N, seed):
    """Rows at every kind of edge of the prefill kernel (256-query tiles, 64-key tiles, the
    sink and window boundaries for sink 4 + window 8192, the prompt's end) plus seeded
    random rows, 24 per head."""
    edges = [0, 1, 3, 4, 5, 63, 64, 255, 256, 4095, 8191, 8192, 8195, 8196, 8197, N // 2, N - 257, N - 256,
             N - 2, N - 1]
    g = np.random.default_rng(seed)
    rnd = sorted(int(x) for x in g.choice(N, size=4, replace=False))
    return sorted(set(edges + rnd))


@pytest.mark.parametrize("N", [32768, 131072])
def test_prefill_bench_configuration_sampled(N):
    """The benchmark's prefill pass (32 query heads over 8 KV heads, retrieval heads
    3, 9, 15, 20, 30, sink 4 + window 8192) at 32K and 128K: 24 rows of every one of the 32
    heads (768 rows), at tile, sink, window and prompt edges and seeded random positions."""
    cfg = W.custom_config(name=f"prefill{N // 1024}k_bench", seed=70 + N // 32768, B=1, Hq=32, Hkv=8, n_ret=5,
                          ret_heads=BENCH_RET, ctx=(N,), window=8192, sinks=4)
    pin = W.make_prefill_inputs(cfg)
    say(f"[gpu] prefill {N}: Hq=32 Hkv=8 ret={BENCH_RET} window=8192 sinks=4")
    out, _ = _run(pin)
    _check_rows(pin, out, [(0, h, _bench_rows(N, 1000 + h)) for h in range(32)])


@pytest.mark.parametrize("B,Hq,Hkv,ret,ctx", [(2, 8, 2, (0, 3, 6), (500, 77)), (1, 4, 4, (2,), (1,))])
def test_prefill_index_keys_bit_exact(B, Hq, Hkv, ret, ctx):
    cfg = W.custom_config(name="prefill_keys", seed=80, B=B, Hq=Hq, Hkv=Hkv, n_ret=len(ret), ret_heads=ret, ctx=ctx)
    pin = W.make_prefill_inputs(cfg)
    say(f"[gpu] prompt index keys B={B} Hq={Hq} Hkv={Hkv} ret={ret} ctx={ctx}")
    t = W.prefill_to_device(pin)
    k_idx = torch.full((B, len(ret), cfg.max_ctx, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    abi.rtp_prefill_index_keys(t["k"], t["w_k"], t["seq_lens"], t["ret_heads"], B, Hq, Hkv, len(ret), cfg.max_ctx,
                               k_idx)
    torch.cuda.synchronize()
    got = k_idx.view(torch.int16).cpu().numpy().view(np.uint16)
    seven = W.f32_to_bf16_bits(np.float32([7.0]))[0]
    G = Hq // Hkv
    for b, n in enumerate(pin.seq_lens):
        for r, h in enumerate(pin.ret_heads):
            want = np.stack([O.index_key(pin.w_k[r], pin.k[b, int(h) // G, i]) for i in range(int(n))])
            assert np.array_equal(got[b, r, :int(n)], want), (b, r)
            assert (got[b, r, int(n):] == seven).all()
