"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and
compare it with the fp64 oracle on the same seeded inputs."""
import sys
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

import workloads as W
from long_context_sparse_amd import DecodeStep, StepShape
from oracle import accept as A
from oracle import rtp_oracle as O


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def shape_of(cfg: W.DecodeConfig, split_tokens: Optional[int] = None) -> StepShape:
    return StepShape(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, n_ret=cfg.n_ret, n_loc=cfg.n_loc, max_ctx=cfg.max_ctx,
                     block=cfg.block, split_tokens=split_tokens or cfg.split_tokens, window=cfg.window,
                     sinks=cfg.sinks)


class Run:
    """One GPU decode step on a workload, with host copies of its outputs."""

    def __init__(self, inp: W.DecodeInputs, tensors=None, split_tokens: Optional[int] = None, tag: str = "",
                 use_mask: bool = True, k_tokens: int = 0, overlap: bool = True):
        cfg = inp.cfg
        self.inp = inp
        self.k_tokens = k_tokens
        say(f"[gpu] {tag or cfg.name}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} n_ret={cfg.n_ret} "
            f"ctx={cfg.ctx[:4]}{'...' if len(cfg.ctx) > 4 else ''} block={cfg.block} "
            f"split={split_tokens or cfg.split_tokens} window={cfg.window} sinks={cfg.sinks} seed={cfg.seed} "
            f"{'masks' if use_mask else 'lists'}{f' top-k {k_tokens}' if k_tokens else ''}")
        self.t = tensors if tensors is not None else W.to_device(inp)
        self.step = DecodeStep(shape_of(cfg, split_tokens), use_mask=use_mask, k_tokens=k_tokens, overlap=overlap)
        self.out = self.step(self.t)
        torch.cuda.synchronize()
        self.out_h = self.out.cpu().numpy().astype(np.float64)
        self.sel_idx = self.step.sel_idx.cpu().numpy()
        self.sel_cnt = self.step.sel_cnt.cpu().numpy()

    def gpu_blocks(self, b: int, r: int) -> np.ndarray:
        return self.sel_idx[b, r, :self.sel_cnt[b, r]]


def check_selection(run: Run, pairs: Optional[Iterable[Tuple[int, int]]] = None) -> Dict[Tuple[int, int], np.ndarray]:
    """Acceptance rule on every (b, r); returns the GPU sets that differ from the oracle's."""
    inp = run.inp
    cfg = inp.cfg
    if pairs is None:
        pairs = [(b, r) for b in range(cfg.B) for r in range(cfg.n_ret)]
    differ = {}
    for b, r in pairs:
        G = run.gpu_blocks(b, r)
        n = int(inp.seq_lens[b])
        nblk = -(-n // cfg.block)
        assert G.size >= 1, (b, r)
        assert np.all(np.diff(G) > 0), f"sel_idx not strictly ascending for {(b, r)}"
        assert G[0] >= 0 and G[-1] < nblk
        m = O.retrieval_masses(inp, b, r)
        p = float(inp.top_p[b, r])
        sel = O.select_top_p(m, p)
        ok, why = A.accept_selection(m, p, G, sel)
        assert ok, f"selection {(b, r)} rejected: {why}"
        if not np.array_equal(G, sel.blocks):
            differ[(b, r)] = G
    return differ


def check_selection_topk(run: Run) -> Dict[Tuple[int, int], np.ndarray]:
    """Static top-k acceptance on every (b, r); returns the GPU sets that differ from the
    oracle's (ties at the threshold)."""
    inp = run.inp
    cfg = inp.cfg
    differ = {}
    for b in range(cfg.B):
        for r in range(cfg.n_ret):
            G = run.gpu_blocks(b, r)
            nblk = -(-int(inp.seq_lens[b]) // cfg.block)
            assert np.all(np.diff(G) > 0), f"sel_idx not strictly ascending for {(b, r)}"
            assert G.size >= 1 and G[0] >= 0 and G[-1] < nblk
            m = O.retrieval_masses(inp, b, r)
            sel = O.select_top_k(m, run.k_tokens, cfg.block)
            ok, why = A.accept_topk(m, run.k_tokens, cfg.block, G, sel)
            assert ok, f"top-k selection {(b, r)} rejected: {why}"
            if not np.array_equal(G, sel.blocks):
                differ[(b, r)] = G
    return differ


def oracle_row(run: Run, b: int, h: int) -> np.ndarray:
    """Oracle output of (b, query head h); retrieval heads attend over the GPU's set
    when it differs from the oracle's but passed the acceptance rule."""
    inp = run.inp
    cfg = inp.cfg
    ret = {int(x): i for i, x in enumerate(inp.ret_heads)}
    n = int(inp.seq_lens[b])
    kv = h // cfg.gqa
    if h in ret:
        r = ret[h]
        blocks = run.gpu_blocks(b, r)
        toks = O.block_tokens(blocks, cfg.block, n)
        return O.attend(inp.q[b, h], inp.k_cache[b, kv], inp.v_cache[b, kv], toks)[0]
    return O.local_head(inp, b, h).out


def check_outputs(run: Run, items: Optional[Sequence[Tuple[int, int]]] = None,
                  max_abs: float = A.TOL_MAX_ABS, mean_rel: float = A.TOL_MEAN_REL) -> Tuple[float, float]:
    cfg = run.inp.cfg
    if items is None:
        items = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    g = np.stack([run.out_h[b, h] for b, h in items])
    o = np.stack([oracle_row(run, b, h) for b, h in items])
    ok, ma, mr = A.outputs_ok(g, o, max_abs, mean_rel)
    say(f"      outputs: {len(items)} rows, max-abs {ma:.3e}, mean-rel {mr:.3e}")
    assert ok, f"outputs out of tolerance: max-abs {ma:.3e} mean-rel {mr:.3e}"
    return ma, mr
