"""The index call's workspace (rtp_index_topp / rtp_index_topk): reuse across batch sizes,
the reported fallback when a bounded wait runs out (forced from the host through the
header's fault-injection word, so every kernel still exits normally), a call with another
number of blocks per sequence, and the wrap of a head's 32-bit call tag.  Block sets are
checked against the oracle's selection (Review, Hardware-aware top-p decoding kernel:
the last workgroup of each head selects, found by an atomic counter)."""
import types

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import check_outputs, check_selection, say
from long_context_sparse_amd import DecodeStep, abi
from gpu_util import shape_of

pytestmark = pytest.mark.gpu

HDR_LAYOUT, HDR_STATUS, HDR_FALLBACKS, HDR_INJECT = 0, 1, 2, 3  # uint32 words of rtp_index_ws_header
WAIT_EXPIRED, LAYOUT_MISMATCH = 1, 2


def _cfg(name, B, n_ret, ctx, seed, max_ctx=None):
    ctx = tuple(ctx)
    if max_ctx is not None:
        ctx = ctx[:-1] + (max_ctx,)  # the last sequence fixes max_ctx
    return W.custom_config(name=name, seed=seed, B=B, Hkv=2, Hq=8, n_ret=n_ret, ctx=ctx, block=64,
                           split_tokens=256, window=64, sinks=4, top_p=tuple([0.9] * n_ret),
                           kind="peaked_diffuse")


class IndexRun:
    """rtp_index_topp on inputs `inp` with a caller-owned workspace; host copies of the sets."""

    def __init__(self, inp, ws, tag):
        cfg = inp.cfg
        self.inp = inp
        t = W.to_device(inp)
        nblk = -(-cfg.max_ctx // cfg.block)
        sel_idx = torch.full((cfg.B, cfg.n_ret, nblk), -7, dtype=torch.int32, device="cuda")
        sel_cnt = torch.zeros((cfg.B, cfg.n_ret), dtype=torch.int32, device="cuda")
        sel_mask = torch.full((cfg.B, cfg.n_ret, nblk), 9, dtype=torch.uint8, device="cuda")
        say(f"[gpu] {tag}: B={cfg.B} n_ret={cfg.n_ret} max_ctx={cfg.max_ctx} nblk={nblk}")
        abi.rtp_index_topp(t["q_pre"], t["w_q"], t["k_idx"], t["seq_lens"], t["ret_heads"], t["top_p"], cfg.B,
                           cfg.Hq, cfg.n_ret, cfg.max_ctx, cfg.block, sel_idx, sel_cnt, ws, sel_mask=sel_mask)
        torch.cuda.synchronize()
        self.sel_idx = sel_idx.cpu().numpy()
        self.sel_cnt = sel_cnt.cpu().numpy()
        self.sel_mask = sel_mask.cpu().numpy()

    def gpu_blocks(self, b, r):
        return self.sel_idx[b, r, :self.sel_cnt[b, r]]

    def all_blocks(self):
        cfg = self.inp.cfg
        for b in range(cfg.B):
            nb = -(-int(self.inp.seq_lens[b]) // cfg.block)
            for r in range(cfg.n_ret):
                if self.sel_cnt[b, r] != nb or not np.array_equal(self.gpu_blocks(b, r), np.arange(nb)):
                    return False
                if not np.all(self.sel_mask[b, r, :nb] == 1):
                    return False
        return True


def _header(ws):
    return ws[:16].view(torch.int32).cpu().numpy().view(np.uint32)


def _set_header(ws, word, value):
    h = ws[:16].view(torch.int32)
    h[word] = int(np.uint32(value).view(np.int32))
    torch.cuda.synchronize()


def test_workspace_serves_smaller_and_larger_batches():
    """One zero-filled workspace sized for 96 heads: 60 heads (B 10), then 96 (B 16), then
    60 again, each against the oracle (the per-head state sits at a fixed stride, so the
    larger batch's counters do not land on the smaller batch's words)."""
    max_ctx = 3000
    ws = torch.zeros(abi.rtp_index_topp_workspace_size(16, 6, max_ctx, 64), dtype=torch.uint8, device="cuda")
    g = np.random.default_rng(4)
    a = W.make_inputs(_cfg("ws_b10", 10, 6, g.integers(1, 3000, size=10), 41, max_ctx))
    b = W.make_inputs(_cfg("ws_b16", 16, 6, g.integers(1, 3000, size=16), 42, max_ctx))
    for inp, tag in ((a, "60 heads"), (b, "96 heads"), (a, "60 heads again")):
        run = IndexRun(inp, ws, tag)
        check_selection(run)
    assert _header(ws)[HDR_STATUS] == 0 and _header(ws)[HDR_FALLBACKS] == 0


def test_forced_wait_expiry_falls_back_to_every_block_and_reports_it():
    """The header's inject bit makes every bounded wait give up: each head then selects
    every block, the status bit and the fallback count report it, every kernel exits, and
    the outputs are the oracle's attention over every block.  With the bit and the status
    cleared, the next step selects as the oracle does (the counters were reset)."""
    cfg = _cfg("ws_inject", 3, 4, (1500, 2900, 64), 43)
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    step = DecodeStep(shape_of(cfg))
    _set_header(step.ws_index, HDR_INJECT, 1)
    say("[gpu] forced wait expiry: step with inject = 1")
    out = step(t)
    torch.cuda.synchronize()
    hdr = _header(step.ws_index)
    assert hdr[HDR_STATUS] & WAIT_EXPIRED
    assert hdr[HDR_FALLBACKS] == cfg.B * cfg.n_ret
    run = types.SimpleNamespace(inp=inp, out_h=out.cpu().numpy().astype(np.float64),
                                sel_idx=step.sel_idx.cpu().numpy(), sel_cnt=step.sel_cnt.cpu().numpy())
    run.gpu_blocks = lambda b, r: run.sel_idx[b, r, :run.sel_cnt[b, r]]
    for b in range(cfg.B):
        nb = -(-int(inp.seq_lens[b]) // cfg.block)
        for r in range(cfg.n_ret):
            assert np.array_equal(run.gpu_blocks(b, r), np.arange(nb)), (b, r)
    check_outputs(run)
    for w in (HDR_INJECT, HDR_STATUS, HDR_FALLBACKS):
        _set_header(step.ws_index, w, 0)
    say("[gpu] forced wait expiry: step after clearing the header")
    out = step(t)
    torch.cuda.synchronize()
    run.out_h = out.cpu().numpy().astype(np.float64)
    run.sel_idx, run.sel_cnt = step.sel_idx.cpu().numpy(), step.sel_cnt.cpu().numpy()
    check_selection(run)
    check_outputs(run)
    hdr = _header(step.ws_index)
    assert hdr[HDR_STATUS] == 0 and hdr[HDR_FALLBACKS] == 0


def test_other_blocks_per_sequence_is_refused_on_the_device():
    """A workspace first used with 47 blocks per sequence, then called with 94: the call
    selects every block, sets the layout-mismatch bit and leaves the state alone; a
    freshly zeroed workspace then serves the second shape normally, and the first shape
    still works on the first workspace."""
    big = abi.rtp_index_topp_workspace_size(4, 4, 6000, 64)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    a = W.make_inputs(_cfg("ws_lay_a", 4, 4, (100, 2999, 1, 3000), 44))
    b = W.make_inputs(_cfg("ws_lay_b", 4, 4, (5000, 64, 6000, 333), 45))
    check_selection(IndexRun(a, ws, "47 blocks"))
    assert _header(ws)[HDR_LAYOUT] == 47
    run = IndexRun(b, ws, "94 blocks on a 47-block workspace")
    assert run.all_blocks()
    hdr = _header(ws)
    assert hdr[HDR_STATUS] == LAYOUT_MISMATCH and hdr[HDR_LAYOUT] == 47 and hdr[HDR_FALLBACKS] == 16
    check_selection(IndexRun(a, ws, "47 blocks again"))
    ws2 = torch.zeros(big, dtype=torch.uint8, device="cuda")
    check_selection(IndexRun(b, ws2, "94 blocks, fresh workspace"))
    assert _header(ws2)[HDR_STATUS] == 0 and _header(ws2)[HDR_LAYOUT] == 94


def test_tag_wrap_clears_the_words():
    """Every head's tag set to 2^32 - 1 (the last before the wrap): that call selects as
    the oracle does, leaves tag 1 and the head's words cleared, and the next call (tag 1)
    selects correctly too."""
    cfg = _cfg("ws_wrap", 2, 3, (2500, 700), 46)
    inp = W.make_inputs(cfg)
    ws = torch.zeros(abi.rtp_index_topp_workspace_size(cfg.B, cfg.n_ret, cfg.max_ctx, cfg.block), dtype=torch.uint8,
                     device="cuda")
    check_selection(IndexRun(inp, ws, "first call"))
    stride = abi.rtp_index_topp_workspace_size(1, 1, cfg.max_ctx, cfg.block) - 256
    heads = cfg.B * cfg.n_ret
    words = ws.view(torch.int32)
    for h in range(heads):
        words[(256 + h * stride) // 4 + 1] = -1  # tag word: 0xFFFFFFFF
    torch.cuda.synchronize()
    check_selection(IndexRun(inp, ws, "call with tag 2^32 - 1"))
    host = ws.cpu().numpy()
    for h in range(heads):
        base = 256 + h * stride
        assert host[base + 4:base + 8].view(np.uint32)[0] == 1, h
        assert not host[base + 256:base + stride].any(), h
        assert host[base:base + 4].view(np.int32)[0] == 0, h  # arrival counter reset
    check_selection(IndexRun(inp, ws, "call with tag 1"))
    assert _header(ws)[HDR_STATUS] == 0


@pytest.mark.parametrize("lens,seed", [
    ((2900, 100, 2900, 1, 1777, 64, 2900, 1, 2900), 46),  # equal lengths: ranked by index
    (tuple(np.random.default_rng(47).integers(1, 300, size=260)), 47),  # over 256: index order
])
def test_ragged_batch_order_serves_every_sequence(lens, seed):
    """The index grid takes sequences longest first (each workgroup ranks the lengths,
    ties by index; batches over 256 sequences keep the index order): every (sequence,
    head) is served exactly once and matches the oracle, with repeated and tiny lengths."""
    B = len(lens)
    cfg = _cfg(f"order_b{B}", B, 2, lens, seed)
    ws = torch.zeros(abi.rtp_index_topp_workspace_size(B, 2, cfg.max_ctx, 64), dtype=torch.uint8, device="cuda")
    inp = W.make_inputs(cfg)
    for tag in ("first call", "second call"):
        run = IndexRun(inp, ws, f"B={B} {tag}")
        check_selection(run)
    assert _header(ws)[HDR_STATUS] == 0 and _header(ws)[HDR_FALLBACKS] == 0
