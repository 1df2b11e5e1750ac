"""GPU parity with retained KV placement: KV groups whose query heads are all local keep
only the sinks and the window, in a ring (Review, Method overview: the non-retrieval
heads drop remote tokens), and the other groups stay in full caches that hold nothing
else.  The step over that placement, and decode loops whose cache appends wrap the
rings, must match the oracle over the full caches; the rings' rows must equal the
placement rule bit for bit."""
import types

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Run, check_outputs, check_selection, say, shape_of
from long_context_sparse_amd import DecodeStep, abi
from oracle import rtp_oracle as O

pytestmark = pytest.mark.gpu

JUNK_K = W.f32_to_bf16_bits(np.float32([30.0]))[0]     # a ring row holding no position:
JUNK_V = W.f32_to_bf16_bits(np.float32([1000.0]))[0]   # any weight on it shows in the output


def ring_row(p: int, sinks: int, window: int) -> int:
    """Ring row of position p (-1: not kept)."""
    if p < sinks:
        return p
    return sinks + (p - sinks) % window if window > 0 else -1


def local_groups(inp) -> list:
    G = inp.cfg.gqa
    ret = {int(h) // G for h in inp.ret_heads}
    return [g for g in range(inp.cfg.Hkv) if g not in ret]


def place(inp, ring_groups, full_order=None):
    """Host-side placement of the inputs: kv_slot, the full caches of the other groups
    (in full_order) and the rings of ring_groups, filled from the first seq_lens rows."""
    cfg = inp.cfg
    S, Wn = cfg.sinks, cfg.window
    full = full_order if full_order is not None else [g for g in range(cfg.Hkv) if g not in ring_groups]
    assert sorted(full + list(ring_groups)) == list(range(cfg.Hkv))
    kv_slot = np.zeros(cfg.Hkv, np.int32)
    for s, g in enumerate(full):
        kv_slot[g] = s
    for j, g in enumerate(ring_groups):
        kv_slot[g] = -1 - j
    kr = np.full((cfg.B, len(ring_groups), S + Wn, 128), JUNK_K, np.uint16)
    vr = np.full((cfg.B, len(ring_groups), S + Wn, 128), JUNK_V, np.uint16)
    for b in range(cfg.B):
        n = int(inp.seq_lens[b])
        keep = O.local_tokens(n, Wn, S)
        for j, g in enumerate(ring_groups):
            rows = [ring_row(int(p), S, Wn) for p in keep]
            kr[b, j, rows] = inp.k_cache[b, g, keep]
            vr[b, j, rows] = inp.v_cache[b, g, keep]
    return dict(kv_slot=kv_slot, k_full=inp.k_cache[:, full], v_full=inp.v_cache[:, full], k_ring=kr, v_ring=vr)


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).cuda()


def placed_tensors(inp, pl):
    t = W.to_device(inp)
    t["k_cache"], t["v_cache"] = _bf(pl["k_full"]), _bf(pl["v_full"])
    t["k_ring"], t["v_ring"] = _bf(pl["k_ring"]), _bf(pl["v_ring"])
    t["kv_slot"] = torch.from_numpy(pl["kv_slot"]).cuda()
    return t


def _host(x):
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


CASES = {
    # G = 4; retrieval heads in groups 0 and 2, groups 1 and 3 in rings; one sequence
    # shorter than sinks + window, one that has wrapped, one long
    "mixed": dict(seed=41, B=3, Hkv=4, Hq=16, n_ret=4, ret_heads=(0, 1, 8, 10), ctx=(5000, 40, 1500),
                  window=1024, sinks=4, split_tokens=1024),
    # no retrieval heads: every group in a ring, no full caches at all
    "all_ring": dict(seed=42, B=2, Hkv=2, Hq=8, n_ret=0, ret_heads=(), ctx=(3000, 9), window=256, sinks=4,
                     split_tokens=256),
    # sinks only (window 0) and window only (no sinks)
    "sinks_only": dict(seed=43, B=2, Hkv=2, Hq=4, n_ret=1, ret_heads=(0,), ctx=(700, 3), window=0, sinks=8,
                       split_tokens=256),
    "window_only": dict(seed=44, B=2, Hkv=4, Hq=8, n_ret=2, ret_heads=(2, 3), ctx=(2049, 100), window=64,
                        sinks=0, split_tokens=512),
    # one query head per KV head, and eight
    "gqa1": dict(seed=46, B=2, Hkv=4, Hq=4, n_ret=1, ret_heads=(2,), ctx=(1500, 70), window=128, sinks=4,
                 split_tokens=512),
    "gqa8": dict(seed=47, B=1, Hkv=2, Hq=16, n_ret=2, ret_heads=(3, 5), ctx=(4000,), window=512, sinks=4,
                 split_tokens=1024),
}


@pytest.mark.parametrize("name", list(CASES))
def test_ring_step_matches_oracle(name):
    cfg = W.custom_config(name=f"ring_{name}", **CASES[name])
    inp = W.make_inputs(cfg)
    rings = local_groups(inp)
    full = [g for g in range(cfg.Hkv) if g not in rings][::-1]   # full slots in reverse order
    pl = place(inp, rings, full)
    say(f"[gpu] ring step {name}: ring groups {rings}, full slots {full}")
    run = Run(inp, tensors=placed_tensors(inp, pl), tag=f"ring {name}")
    if cfg.n_ret:
        check_selection(run)
    check_outputs(run)


def test_ring_step_static_topk():
    """The ring placement under the static top-k rule (a 256-token budget)."""
    from gpu_util import check_selection_topk
    cfg = W.custom_config(name="ring_topk", **CASES["mixed"])
    inp = W.make_inputs(cfg)
    rings = local_groups(inp)
    run = Run(inp, tensors=placed_tensors(inp, place(inp, rings)), tag="ring top-k 256", k_tokens=256)
    check_selection_topk(run)
    check_outputs(run)


def test_ring_step_full_size():
    """A 128K-token batch of four with half the KV groups in rings: every local head of
    the ring groups and every retrieval head against the oracle; sampled outputs only."""
    cfg = W.custom_config(name="ctx128k_ring", seed=3, B=4, Hkv=8, Hq=32, n_ret=8, ctx=(131072,) * 4, block=64,
                          top_p=(0.95,) * 8, window=8192, sinks=4, split_tokens=1024, kind="peaked_diffuse",
                          ret_heads=(0, 1, 4, 5, 8, 9, 12, 13))
    inp = W.make_inputs(cfg)
    rings = local_groups(inp)
    assert rings == [4, 5, 6, 7]
    run = Run(inp, tensors=placed_tensors(inp, place(inp, rings)), tag="ctx128k ring")
    check_selection(run)
    items = [(b, h) for b in range(cfg.B) for h in range(16, 32, 3)]
    items += [(b, int(h)) for b in (0, 3) for h in inp.ret_heads]
    check_outputs(run, items)


@pytest.mark.parametrize("window,sinks,steps", [(32, 4, 45), (16, 0, 20), (0, 5, 8)])
def test_decode_loop_with_appends(window, sinks, steps):
    """Decode loop: each step appends one token (K/V rows to the full cache or the ring,
    index keys of the retrieval heads), takes a new query and runs the step.  The rings
    wrap more than once; every step's outputs match the oracle over the full caches."""
    B, Hkv, Hq, n_ret = 2, 2, 8, 2
    n0 = (300, 30)
    cfg = W.custom_config(name="ring_loop", seed=45 + window, B=B, Hkv=Hkv, Hq=Hq, n_ret=n_ret, ret_heads=(0, 2),
                          ctx=tuple(n + steps for n in n0), window=window, sinks=sinks, split_tokens=128)
    inp = W.make_inputs(cfg)
    G = cfg.gqa
    inp.seq_lens[:] = n0
    rings = local_groups(inp)
    assert rings == [1]
    pl = place(inp, rings)
    for b, n in enumerate(n0):                      # rows past the sequences: junk until appended
        pl["k_full"][b, :, n:] = JUNK_K
        pl["v_full"][b, :, n:] = JUNK_V
    t = placed_tensors(inp, pl)
    step = DecodeStep(shape_of(cfg))
    w_k = _bf(inp.w_k)
    g = np.random.default_rng(7 + window)
    say(f"[gpu] ring decode loop window={window} sinks={sinks} steps={steps}")
    for i in range(steps):
        inp.seq_lens += 1
        lens = [int(n) for n in inp.seq_lens]
        k_new = np.stack([inp.k_cache[b, :, n - 1] for b, n in enumerate(lens)])
        v_new = np.stack([inp.v_cache[b, :, n - 1] for b, n in enumerate(lens)])
        inp.q[:] = W.f32_to_bf16_bits(g.standard_normal(inp.q.shape, dtype=np.float32))
        for b, n in enumerate(lens):                  # the oracle sees the appended index keys
            for r, h in enumerate(inp.ret_heads):
                inp.k_idx[b, r, n - 1] = O.index_key(inp.w_k[r], k_new[b, int(h) // G])
        t["seq_lens"].copy_(torch.from_numpy(inp.seq_lens.astype(np.int32)))
        t["q"].copy_(_bf(inp.q))
        abi.rtp_cache_append(_bf(k_new), _bf(v_new), _bf(k_new), w_k, t["seq_lens"], t["ret_heads"], B, Hq, Hkv,
                             n_ret, cfg.max_ctx, t["k_cache"], t["v_cache"], t["k_idx"], sinks=sinks, window=window,
                             **DecodeStep.placement(t))
        out = step(t)
        torch.cuda.synchronize()
        run = types.SimpleNamespace(inp=inp, out_h=out.cpu().numpy().astype(np.float64),
                                    sel_idx=step.sel_idx.cpu().numpy(), sel_cnt=step.sel_cnt.cpu().numpy())
        run.gpu_blocks = lambda b, r, run=run: run.sel_idx[b, r, :run.sel_cnt[b, r]]
        check_selection(run)
        check_outputs(run)
    # the rings and the full caches hold exactly what the placement rule says
    want = place(inp, rings)
    kr, vr = _host(t["k_ring"]), _host(t["v_ring"])
    for b, n in enumerate(inp.seq_lens):
        rows = sorted({ring_row(int(p), sinks, window) for p in O.local_tokens(int(n), window, sinks)})
        assert np.array_equal(kr[b, :, rows], want["k_ring"][b, :, rows])
        assert np.array_equal(vr[b, :, rows], want["v_ring"][b, :, rows])
    kf, vf = _host(t["k_cache"]), _host(t["v_cache"])
    for b, n in enumerate(inp.seq_lens):
        assert np.array_equal(kf[b, :, :n], want["k_full"][b, :, :n])
        assert np.array_equal(vf[b, :, :n], want["v_full"][b, :, :n])




@pytest.mark.parametrize("name", list(CASES))
def test_ring_fill_matches_placement(name):
    """rtp_ring_fill from the prompt's full K/V gives the placement rule's ring rows bit
    for bit; rows no position maps to keep what they held."""
    cfg = W.custom_config(name=f"ring_{name}", **CASES[name])
    inp = W.make_inputs(cfg)
    rings = local_groups(inp)
    pl = place(inp, rings)
    say(f"[gpu] ring fill {name}: ring groups {rings}")
    kr = torch.full(pl["k_ring"].shape, 3.0, dtype=torch.bfloat16, device="cuda")
    vr = torch.full(pl["v_ring"].shape, 3.0, dtype=torch.bfloat16, device="cuda")
    t = W.to_device(inp)
    abi.rtp_ring_fill(t["k_cache"], t["v_cache"], t["seq_lens"], torch.from_numpy(pl["kv_slot"]).cuda(), cfg.B,
                      cfg.Hkv, cfg.max_ctx, kr, vr, len(rings), cfg.sinks, cfg.window)
    torch.cuda.synchronize()
    got_k, got_v = _host(kr), _host(vr)
    three = W.f32_to_bf16_bits(np.float32([3.0]))[0]
    for b, n in enumerate(inp.seq_lens):
        held = sorted({ring_row(int(p), cfg.sinks, cfg.window) for p in O.local_tokens(int(n), cfg.window, cfg.sinks)})
        empty = [r for r in range(cfg.sinks + cfg.window) if r not in held]
        assert np.array_equal(got_k[b, :, held], pl["k_ring"][b, :, held])
        assert np.array_equal(got_v[b, :, held], pl["v_ring"][b, :, held])
        assert (got_k[b, :, empty] == three).all() and (got_v[b, :, empty] == three).all()


def test_prefill_then_decode():
    """The whole cache life cycle on the device: the prompt's index keys
    (rtp_prefill_index_keys) and rings (rtp_ring_fill) from its K/V, then decode steps
    that append tokens and wrap the rings; every step against the oracle over the full
    caches, whose prompt index keys the oracle computes itself."""
    B, Hkv, Hq, n_ret, steps, window, sinks = 2, 2, 8, 2, 40, 32, 4
    n0 = (300, 30)
    cfg = W.custom_config(name="prefill_decode", seed=77, B=B, Hkv=Hkv, Hq=Hq, n_ret=n_ret, ret_heads=(0, 2),
                          ctx=tuple(n + steps for n in n0), window=window, sinks=sinks, split_tokens=128)
    inp = W.make_inputs(cfg)
    G = cfg.gqa
    inp.seq_lens[:] = n0
    say(f"[gpu] prefill then decode: prompts {n0}, {steps} steps, window {window} sinks {sinks}")
    for b, n in enumerate(n0):                         # the oracle's own prompt index keys
        for r, h in enumerate(inp.ret_heads):
            for i in range(n):
                inp.k_idx[b, r, i] = O.index_key(inp.w_k[r], inp.k_cache[b, int(h) // G, i])
    full = W.to_device(inp)                            # the prompt's K/V of every group
    rings = local_groups(inp)
    assert rings == [1]
    kv_slot = torch.tensor([0, -1], dtype=torch.int32, device="cuda")
    k_idx = torch.full_like(full["k_idx"], 5.0)
    abi.rtp_prefill_index_keys(full["k_cache"], _bf(inp.w_k), full["seq_lens"], full["ret_heads"], B, Hq, Hkv, n_ret,
                               cfg.max_ctx, k_idx)
    kr = torch.zeros((B, 1, sinks + window, 128), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros_like(kr)
    abi.rtp_ring_fill(full["k_cache"], full["v_cache"], full["seq_lens"], kv_slot, B, Hkv, cfg.max_ctx, kr, vr, 1,
                      sinks, window)
    torch.cuda.synchronize()
    ki = _host(k_idx)
    for b, n in enumerate(n0):
        assert np.array_equal(ki[b, :, :n], inp.k_idx[b, :, :n]), b
    # decode state: group 0 keeps a full cache (its prompt rows, junk past them), group 1 its ring
    kc = full["k_cache"][:, :1].clone()
    vc = full["v_cache"][:, :1].clone()
    for b, n in enumerate(n0):
        kc[b, :, n:] = 30.0
        vc[b, :, n:] = 1000.0
    t = dict(full)
    t.update(k_cache=kc, v_cache=vc, k_idx=k_idx, kv_slot=kv_slot, k_ring=kr, v_ring=vr)
    step = DecodeStep(shape_of(cfg))
    w_k = _bf(inp.w_k)
    g = np.random.default_rng(78)
    for i in range(steps):
        inp.seq_lens += 1
        lens = [int(n) for n in inp.seq_lens]
        k_new = np.stack([inp.k_cache[b, :, n - 1] for b, n in enumerate(lens)])
        v_new = np.stack([inp.v_cache[b, :, n - 1] for b, n in enumerate(lens)])
        inp.q[:] = W.f32_to_bf16_bits(g.standard_normal(inp.q.shape, dtype=np.float32))
        for b, n in enumerate(lens):
            for r, h in enumerate(inp.ret_heads):
                inp.k_idx[b, r, n - 1] = O.index_key(inp.w_k[r], k_new[b, int(h) // G])
        t["seq_lens"].copy_(torch.from_numpy(inp.seq_lens.astype(np.int32)))
        t["q"].copy_(_bf(inp.q))
        abi.rtp_cache_append(_bf(k_new), _bf(v_new), _bf(k_new), w_k, t["seq_lens"], t["ret_heads"], B, Hq, Hkv,
                             n_ret, cfg.max_ctx, t["k_cache"], t["v_cache"], t["k_idx"], sinks=sinks, window=window,
                             **DecodeStep.placement(t))
        out = step(t)
        torch.cuda.synchronize()
        run = types.SimpleNamespace(inp=inp, out_h=out.cpu().numpy().astype(np.float64),
                                    sel_idx=step.sel_idx.cpu().numpy(), sel_cnt=step.sel_cnt.cpu().numpy())
        run.gpu_blocks = lambda b, r, run=run: run.sel_idx[b, r, :run.sel_cnt[b, r]]
        check_selection(run)
        check_outputs(run)
