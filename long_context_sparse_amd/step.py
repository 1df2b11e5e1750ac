"""One decode step of the sparse attention path, as one librtp call (three launches).

DecodeStep owns the device buffers the calls need (selected-block lists and masks,
split partials, workspaces, output) and issues them through one rtp_decode_step call,
three launches on the current stream (the local heads' part on a second stream when
their bytes are comparable to the index keys'):

  rtp_index_topp (or rtp_index_topk)   retrieval heads: scores and block selection
  rtp_decode_attn                      retrieval heads' split attention + local heads' window
  rtp_decode_merge                     both kinds of partials -> the output rows

The four separate calls of the path (rtp_index_topp, rtp_sparse_attn_split,
rtp_split_reduce, rtp_local_window_attn) stay available one by one.

The inputs may place KV groups in sink + window rings (keys "kv_slot", "k_ring",
"v_ring"; see the KV placement note in include/rtp.h): the full caches then hold only
the groups with kv_slot >= 0.

PyTorch provides the memory and the streams; every step runs in librtp.so.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

from . import abi

HEAD_DIM = 128
INDEX_DIM = 16


@dataclasses.dataclass(frozen=True)
class StepShape:
    B: int
    Hq: int
    Hkv: int
    n_ret: int
    n_loc: int
    max_ctx: int
    block: int
    split_tokens: int
    window: int
    sinks: int

    @property
    def nblk_max(self) -> int:
        return -(-self.max_ctx // self.block)

    @property
    def n_split(self) -> int:
        return -(-self.max_ctx // self.split_tokens)


class DecodeStep:
    def __init__(self, shape: StepShape, device: str = "cuda", use_mask: bool = True, k_tokens: int = 0,
                 overlap: bool = True):
        """k_tokens = 0: the top-p rule (the inputs' top_p); > 0: the static top-k rule
        with this budget in tokens.  overlap: give rtp_decode_step a second stream and two
        events, which it uses when the local heads' bytes are comparable to the index
        keys' (False: one stream always)."""
        self.s = shape
        self.k_tokens = int(k_tokens)
        dev = torch.device(device)
        self.device = dev
        s = shape
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.sel_idx = torch.zeros((s.B, max(s.n_ret, 1), s.nblk_max), **i32)
        self.sel_cnt = torch.zeros((s.B, max(s.n_ret, 1)), **i32)
        # per-head block masks: the index call writes them and the split attention reads
        # its union from them in one round of loads (use_mask=False: the lists are searched)
        self.sel_mask = (torch.zeros((s.B, max(s.n_ret, 1), s.nblk_max), dtype=torch.uint8, device=dev)
                         if use_mask else None)
        self.o_part = torch.zeros((s.B, max(s.n_ret, 1), s.n_split, HEAD_DIM), **f32)
        self.lse_part = torch.zeros((s.B, max(s.n_ret, 1), s.n_split), **f32)
        self.out = torch.zeros((s.B, s.Hq, HEAD_DIM), **f32)
        ws1 = abi.rtp_index_topp_workspace_size(s.B, s.n_ret, s.max_ctx, s.block) if s.n_ret else 0
        ws2 = (abi.rtp_local_window_workspace_size(s.B, s.Hq, s.Hkv, s.n_loc, s.max_ctx, s.window, s.sinks)
               if s.n_loc else 0)
        self.ws_index = torch.zeros(max(ws1, 256), dtype=torch.uint8, device=dev)
        self.ws_local = torch.zeros(max(ws2, 256), dtype=torch.uint8, device=dev)
        self.overlap = overlap and s.n_loc > 0 and s.n_ret > 0
        self.side = torch.cuda.Stream(device=dev) if self.overlap else None
        self._fork = abi.event_create(abi.EVENT_DEVICE_ORDER) if self.overlap else None
        self._join = abi.event_create(abi.EVENT_DEVICE_ORDER) if self.overlap else None
        self._key = None
        self._vals = None
        self._step_fn = abi.lib().rtp_decode_step

    @staticmethod
    def placement(t: Dict[str, torch.Tensor]) -> dict:
        """KV placement arguments of these inputs: none (every group in the full caches)
        unless they carry a kv_slot table and the ring caches."""
        if t.get("kv_slot") is None:
            return dict(kv_slot=None, n_full=0, k_ring=None, v_ring=None, n_ring=0)
        return dict(kv_slot=t["kv_slot"], n_full=int(t["k_cache"].shape[1]), k_ring=t["k_ring"],
                    v_ring=t["v_ring"], n_ring=int(t["k_ring"].shape[1]))

    # -- the four calls -------------------------------------------------------------
    def index_topk(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_index_topk(t["q_pre"], t["w_q"], t["k_idx"], t["seq_lens"], t["ret_heads"], self.k_tokens,
                           s.B, s.Hq, s.n_ret, s.max_ctx, s.block, self.sel_idx, self.sel_cnt, self.ws_index,
                           stream, sel_mask=self.sel_mask)

    def index_topp(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_index_topp(t["q_pre"], t["w_q"], t["k_idx"], t["seq_lens"], t["ret_heads"], t["top_p"],
                           s.B, s.Hq, s.n_ret, s.max_ctx, s.block, self.sel_idx, self.sel_cnt,
                           self.ws_index, stream, sel_mask=self.sel_mask)

    def sparse_attn(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_sparse_attn_split(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], t["ret_heads"],
                                  self.sel_idx, self.sel_cnt, s.B, s.Hq, s.Hkv, s.n_ret, s.max_ctx,
                                  s.block, s.split_tokens, self.o_part, self.lse_part, stream,
                                  sel_mask=self.sel_mask, kv_slot=t.get("kv_slot"),
                                  n_full=self.placement(t)["n_full"])

    def reduce(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_split_reduce(self.o_part, self.lse_part, t["ret_heads"], s.B, s.Hq, s.n_ret, s.n_split,
                             self.out, stream)

    # -- the step's own launches after the index call ---------------------------------
    def attn(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_decode_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"],
                            t["ret_heads"] if s.n_ret else None, self.sel_idx if s.n_ret else None,
                            self.sel_cnt if s.n_ret else None, self.sel_mask if s.n_ret else None,
                            t["loc_heads"] if s.n_loc else None, s.B, s.Hq, s.Hkv, s.n_ret, s.n_loc, s.max_ctx,
                            s.block, s.split_tokens, s.window, s.sinks, self.o_part, self.lse_part, self.ws_local,
                            stream, **self.placement(t))

    def merge(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_decode_merge(self.o_part, self.lse_part, t["ret_heads"] if s.n_ret else None,
                             t["loc_heads"] if s.n_loc else None, s.B, s.Hq, s.Hkv, s.n_ret, s.n_loc, s.max_ctx,
                             s.split_tokens, s.window, s.sinks, self.ws_local, self.out, stream)

    def local(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_local_window_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], t["loc_heads"],
                                  s.B, s.Hq, s.Hkv, s.n_loc, s.max_ctx, s.window, s.sinks, self.out,
                                  self.ws_local, stream, **self.placement(t))

    # -- the whole step -------------------------------------------------------------
    def _plan(self, t: Dict[str, torch.Tensor], main: int) -> tuple:
        """Arguments of rtp_decode_step for these tensors and this stream, converted once
        (the C function takes raw pointers and sizes)."""
        s = self.s
        p = abi.device_ptr
        z = lambda name: p(t[name]) if t[name].numel() else None  # noqa: E731
        side = self.side.cuda_stream if self.overlap else None
        pl = self.placement(t)
        o = lambda x: None if x is None else p(x)  # noqa: E731
        return (z("q_pre") if s.n_ret else None, z("w_q") if s.n_ret else None, z("k_idx") if s.n_ret else None,
                p(t["q"]), p(t["k_cache"]), p(t["v_cache"]), p(t["seq_lens"]),
                z("ret_heads") if s.n_ret else None, z("loc_heads") if s.n_loc else None,
                z("top_p") if s.n_ret else None, self.k_tokens, s.B, s.Hq, s.Hkv, s.n_ret, s.n_loc, s.max_ctx, s.block,
                s.split_tokens, s.window, s.sinks, p(self.sel_idx), p(self.sel_cnt),
                p(self.sel_mask) if self.sel_mask is not None else None, p(self.o_part), p(self.lse_part),
                p(self.out), p(self.ws_index), abi.nbytes(self.ws_index), p(self.ws_local),
                abi.nbytes(self.ws_local), o(pl["kv_slot"]), pl["n_full"], o(pl["k_ring"]), o(pl["v_ring"]),
                pl["n_ring"], main, side, self._fork, self._join)

    def __call__(self, t: Dict[str, torch.Tensor]) -> torch.Tensor:
        """Enqueue one decode step on the current stream; returns the fp32 [B, Hq, 128] output.

        One rtp_decode_step call (three launches on that stream).  The arguments are
        converted once per (set of tensors, stream)."""
        main = torch.cuda.current_stream(self.device).cuda_stream
        vals = tuple(t.values())
        key = (main,) + tuple(map(id, vals))
        if self._key != key:
            self._args = self._plan(t, main)
            self._key = key
            self._vals = vals  # the plan's tensors stay alive, so their ids stay theirs
        abi.check("rtp_decode_step", self._step_fn(*self._args))
        return self.out
