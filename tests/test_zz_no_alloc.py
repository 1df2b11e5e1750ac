"""rtp_decode_step_noalloc (workspaces and split partials in the library's fixed device
scratch) against rtp_decode_step (caller-owned workspaces) on the same inputs: the
selected blocks, their masks and the outputs must be bit-identical.  Three calls in a row
on one device: a batch, a smaller batch with fewer blocks per sequence (the scratch's
index part is cleared again), then the first batch once more."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, shape_of
from long_context_sparse_amd import DecodeStep, abi

pytestmark = pytest.mark.gpu


def _cfg(name, B, n_ret, ctx, seed):
    return W.custom_config(name=name, seed=seed, B=B, Hkv=2, Hq=8, n_ret=n_ret, ctx=tuple(ctx), block=64,
                           split_tokens=256, window=256, sinks=4, top_p=tuple([0.9] * n_ret), kind="peaked_diffuse")


def _compare(cfg):
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    say(f"[gpu] no-alloc step {cfg.name}: B={cfg.B} n_ret={cfg.n_ret} max_ctx={cfg.max_ctx}")
    ref = DecodeStep(shape_of(cfg))
    out_ref = ref(t).clone()
    torch.cuda.synchronize()
    s = shape_of(cfg)
    nblk = -(-s.max_ctx // s.block)
    sel_idx = torch.full((s.B, s.n_ret, nblk), -3, dtype=torch.int32, device="cuda")
    sel_cnt = torch.zeros((s.B, s.n_ret), dtype=torch.int32, device="cuda")
    sel_mask = torch.zeros((s.B, s.n_ret, nblk), dtype=torch.uint8, device="cuda")
    out = torch.full((s.B, s.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    abi.rtp_decode_step_noalloc(t["q_pre"], t["w_q"], t["k_idx"], t["q"], t["k_cache"], t["v_cache"], t["seq_lens"],
                                t["ret_heads"], t["loc_heads"], t["top_p"], 0, s.B, s.Hq, s.Hkv, s.n_ret, s.n_loc,
                                s.max_ctx, s.block, s.split_tokens, s.window, s.sinks, sel_idx, sel_cnt, sel_mask,
                                out)
    torch.cuda.synchronize()
    assert torch.equal(sel_cnt, ref.sel_cnt)
    for b in range(s.B):
        for r in range(s.n_ret):
            c = int(sel_cnt[b, r])
            assert torch.equal(sel_idx[b, r, :c], ref.sel_idx[b, r, :c]), (b, r)
            n = -(-int(inp.seq_lens[b]) // s.block)
            assert torch.equal(sel_mask[b, r, :n], ref.sel_mask[b, r, :n]), (b, r)
    assert torch.equal(out, out_ref), float((out - out_ref).abs().max())


def test_noalloc_step_matches_the_step_with_workspaces():
    assert abi.rtp_decode_step_noalloc_limit() == 32 << 20
    g = np.random.default_rng(12)
    a = _cfg("noalloc_a", 3, 3, (3000, 777, 2048), 61)
    b = _cfg("noalloc_b", 2, 2, (1500, 64), 62)       # smaller: fewer sequences, heads and blocks
    _compare(a)
    _compare(b)
    _compare(a)
    del g


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """Sizes whose partials exceed the fixed 8 MiB share: RTP_ESCRATCH, nothing enqueued."""
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    B, Hq, Hkv, n_ret, max_ctx = 64, 32, 8, 32, 1 << 20
    with pytest.raises(abi.RTPError) as e:
        abi.rtp_decode_step_noalloc(x, x, x, x, x, x, x, x, x, x, 0, B, Hq, Hkv, n_ret, 0, max_ctx, 128, 128, 0, 4,
                                    x, x, None, x)
    assert e.value.status == abi.RTP_ESCRATCH
