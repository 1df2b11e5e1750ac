"""Seeded random sweeps of small shapes, decode step and prefill, against the oracle:
head groupings 1-8, any number of retrieval heads (none to all), ragged lengths down to
one token, block 64 or 128, split sizes of 1-16 blocks, windows from 0 to past the
context, 0-9 sinks, top-p from 0.5 to 1 or a static top-k budget of 1-5000 tokens."""
import numpy as np
import pytest

import workloads as W
from gpu_util import Run, check_outputs, check_selection, check_selection_topk, say
from test_gpu_prefill import _check_rows, _run as _prefill_run

pytestmark = pytest.mark.gpu


def _decode_cases(n, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(g.choice([1, 2, 4]))
        G = int(g.choice([1, 2, 4, 8]))
        Hq = Hkv * G
        n_ret = int(g.integers(0, Hq + 1))
        B = int(g.integers(1, 4))
        ctx = tuple(int(x) for x in g.integers(1, 3001, size=B))
        block = int(g.choice([64, 128]))
        split = block * int(g.choice([1, 2, 4, 8, 16]))
        window = int(g.choice([0, 1, 17, 256, 4096]))
        sinks = int(g.choice([0, 1, 4, 9]))
        if window + sinks == 0:
            sinks = 1
        top_p = tuple(float(x) for x in g.choice([0.5, 0.9, 0.99, 1.0], size=n_ret))
        kind = str(g.choice(["random", "peaked_diffuse"]))
        k_tokens = int(g.choice([0, 0, 1, 200, 1000, 5000]))  # 0: top-p; else the static top-k budget
        out.append(dict(name=f"rand{i}", seed=100 + i, B=B, Hkv=Hkv, Hq=Hq, n_ret=n_ret, ctx=ctx, block=block,
                        split_tokens=split, window=window, sinks=sinks, top_p=top_p, kind=kind, k_tokens=k_tokens))
    return out


def _prefill_cases(n, seed=2025):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(g.choice([1, 2]))
        G = int(g.choice([1, 2, 4, 8]))
        Hq = Hkv * G
        n_ret = int(g.integers(0, Hq + 1))
        ret = tuple(sorted(int(x) for x in g.choice(Hq, size=n_ret, replace=False)))
        B = int(g.integers(1, 3))
        ctx = tuple(int(x) for x in g.integers(1, 1501, size=B))
        window = int(g.choice([0, 1, 5, 64, 700, 5000]))
        sinks = int(g.choice([0, 1, 4]))
        if window + sinks == 0:
            window = 1
        out.append(dict(name=f"prand{i}", seed=200 + i, B=B, Hkv=Hkv, Hq=Hq, n_ret=n_ret, ret_heads=ret, ctx=ctx,
                        window=window, sinks=sinks))
    return out


DECODE = _decode_cases(40)
PREFILL = _prefill_cases(24)


@pytest.mark.parametrize("spec", DECODE, ids=[c["name"] for c in DECODE])
def test_random_decode_shapes(spec):
    spec = dict(spec)
    name = spec.pop("name")
    k_tokens = spec.pop("k_tokens")
    cfg = W.custom_config(name=name, **spec)
    run = Run(W.make_inputs(cfg), tag=f"{name} {spec}", k_tokens=k_tokens)
    if cfg.n_ret:
        (check_selection_topk if k_tokens else check_selection)(run)
    check_outputs(run)


@pytest.mark.parametrize("spec", PREFILL, ids=[c["name"] for c in PREFILL])
def test_random_prefill_shapes(spec):
    spec = dict(spec)
    name = spec.pop("name")
    cfg = W.custom_config(name=name, **spec)
    pin = W.make_prefill_inputs(cfg, pad_value=W.BF16_NAN)
    say(f"[gpu] prefill {name}: {spec}")
    out, _ = _prefill_run(pin)
    items = [(b, h, list(range(int(n)))) for b, n in enumerate(pin.seq_lens) for h in range(cfg.Hq)]
    _check_rows(pin, out, items)
