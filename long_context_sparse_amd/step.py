"""One decode step of the sparse attention path, as four librtp calls.

DecodeStep owns the device buffers the calls need (selected-block lists, split
partials, workspaces, output) and issues

  retrieval heads:  rtp_index_topp -> rtp_sparse_attn_split -> rtp_split_reduce
  local heads:      rtp_local_window_attn (on a second stream, overlapping the above)

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
    def __init__(self, shape: StepShape, device: str = "cuda", overlap: bool = True):
        self.s = shape
        dev = torch.device(device)
        self.device = dev
        s = shape
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.sel_idx = torch.zeros((s.B, max(s.n_ret, 1), s.nblk_max), **i32)
        self.sel_cnt = torch.zeros((s.B, max(s.n_ret, 1)), **i32)
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
        self._fork = torch.cuda.Event() if self.overlap else None
        self._join = torch.cuda.Event() if self.overlap else None

    # -- the four calls -------------------------------------------------------------
    def index_topp(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_index_topp(t["q_pre"], t["w_q"], t["k_idx"], t["seq_lens"], t["ret_heads"], t["top_p"],
                           s.B, s.Hq, s.n_ret, s.max_ctx, s.block, self.sel_idx, self.sel_cnt,
                           self.ws_index, stream)

    def sparse_attn(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_sparse_attn_split(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], t["ret_heads"],
                                  self.sel_idx, self.sel_cnt, s.B, s.Hq, s.Hkv, s.n_ret, s.max_ctx,
                                  s.block, s.split_tokens, self.o_part, self.lse_part, stream)

    def reduce(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_split_reduce(self.o_part, self.lse_part, t["ret_heads"], s.B, s.Hq, s.n_ret, s.n_split,
                             self.out, stream)

    def local(self, t: Dict[str, torch.Tensor], stream=None) -> None:
        s = self.s
        abi.rtp_local_window_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], t["loc_heads"],
                                  s.B, s.Hq, s.Hkv, s.n_loc, s.max_ctx, s.window, s.sinks, self.out,
                                  self.ws_local, stream)

    def __call__(self, t: Dict[str, torch.Tensor]) -> torch.Tensor:
        """Enqueue one decode step on the current stream; returns the fp32 [B, Hq, 128] output."""
        main = torch.cuda.current_stream(self.device)
        if self.overlap:
            self._fork.record(main)
            self.side.wait_event(self._fork)
            self.local(t, self.side)
            self._join.record(self.side)
        elif self.s.n_loc:
            self.local(t, main)
        if self.s.n_ret:
            self.index_topp(t, main)
            self.sparse_attn(t, main)
            self.reduce(t, main)
        if self.overlap:
            main.wait_event(self._join)
        return self.out
