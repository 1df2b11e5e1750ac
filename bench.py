"""Decode-step benchmark of the sparse attention path on one MI355X.

One step = the whole hot path for one decode token of every sequence and query
head of a workload, one rtp_decode_step call, three launches on one stream:
rtp_index_topp (scores and block selection of the retrieval heads) -> rtp_decode_attn
(the retrieval heads' block-sparse split attention and the local heads' window attention
in one grid) -> rtp_decode_merge (both kinds of partials -> outputs).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ctx128k]
                    [--also ctx1m,ctx128k@topk4096,mixed,ctx32k,tiny] [--minimal]

A workload name with "@topkK" runs the step with the static top-k rule (a budget of K
tokens, rtp_index_topk) in place of top-p.

Prints ONE JSON line.  `value` is the effective HBM bandwidth of the step,
algorithmic bytes / step latency, with every input resident in HBM before the
timed region.  Algorithmic bytes are what the method must move (index keys of
every cached token of every retrieval head, K/V rows of the union of selected
tokens and window/sink tokens per KV head, queries, projections, outputs),
counted from the block sets the device selected; scratch traffic (block LSEs,
split partials) is excluded.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time
from typing import Dict, List, Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-decode step latency (µs) + effective HBM GB/s at 128K and 1M ctx"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
KERNEL_NAMES = {                # launch of the step -> its kernel
    "index_topp": "index_topp_kernel",
    "index_topk": "index_topp_kernel",
    "decode_attn": "step_attn_kernel",
    "decode_merge": "merge_step_kernel",
}


CALL_NAMES = {"index_topp": "rtp_index_topp", "index_topk": "rtp_index_topk", "decode_attn": "rtp_decode_attn",
              "decode_merge": "rtp_decode_merge"}


def log(*a) -> None:
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic bytes
def block_token_mask(blocks: np.ndarray, block: int, n: int) -> np.ndarray:
    m = np.zeros(n, dtype=bool)
    for j in blocks.tolist():
        m[j * block:min(n, (j + 1) * block)] = True
    return m


def local_token_mask(n: int, window: int, sinks: int) -> np.ndarray:
    m = np.zeros(n, dtype=bool)
    m[:min(sinks, n)] = True
    m[max(0, n - window):n] = True
    return m


def algorithmic_bytes(cfg, inp, sel_idx: np.ndarray, sel_cnt: np.ndarray) -> Dict[str, float]:
    """Bytes each launch of the step (and the whole step) must move for the given block
    selection.

    index_topp:   W^Q (4 KiB a retrieval head) + 32 B per cached token per retrieval
                  head (16 bf16 index dims) + the q_pre row + the selected-block list.
    decode_attn:  512 B (K and V rows, 128 bf16 each) per (KV head, token) in the union,
                  over the group's heads, of the retrieval heads' selected blocks and (for
                  groups with local heads) the sinks + window, + every query row (256 B).
    decode_merge: the fp32 output rows (512 B) of every query head.
    step:         the sum.  Partials (split and window) are scratch and not counted.
    """
    G = cfg.Hq // cfg.Hkv
    ret = [int(h) for h in inp.ret_heads]
    loc = [int(h) for h in inp.loc_heads]
    out = dict(index_topp=0.0, decode_attn=0.0, decode_merge=0.0, step=0.0)
    out["index_topp"] += len(ret) * 16 * 128 * 2
    kv_sel = kv_win = 0
    for b in range(cfg.B):
        n = int(inp.seq_lens[b])
        for r in range(len(ret)):
            out["index_topp"] += 32.0 * n + 256 + 4 * int(sel_cnt[b, r]) + 4
        out["decode_attn"] += 256.0 * (len(ret) + len(loc))
        out["decode_merge"] += 512.0 * (len(ret) + len(loc))
        for g in range(cfg.Hkv):
            rs = [r for r, h in enumerate(ret) if h // G == g]
            has_loc = any(h // G == g for h in loc)
            sel = np.zeros(n, dtype=bool)
            for r in rs:
                sel |= block_token_mask(sel_idx[b, r, :int(sel_cnt[b, r])], cfg.block, n)
            win = local_token_mask(n, cfg.window, cfg.sinks) if has_loc else np.zeros(n, dtype=bool)
            out["decode_attn"] += 512.0 * int((sel | win).sum())
            kv_sel += int(sel.sum())
            kv_win += int(win.sum())
    out["step"] = out["index_topp"] + out["decode_attn"] + out["decode_merge"]
    out["kv_tokens_selected"] = float(sum(int(sel_cnt[b, r]) for b in range(cfg.B) for r in range(len(ret))))
    out["kv_rows_selected_union"] = float(kv_sel)
    out["kv_rows_window"] = float(kv_win)
    return out


# ------------------------------------------------------------------ traffic records
KERNEL_SOURCE = {"index_topp_kernel": "index_topp.hip", "step_attn_kernel": "sparse_attn.hip",
                 "merge_step_kernel": "sparse_attn.hip", "sparse_attn_kernel": "sparse_attn.hip",
                 "merge_kernel": "sparse_attn.hip", "local_window_kernel": "sparse_attn.hip",
                 "prefill_kernel": "prefill_attn.hip"}


def kernel_source_hash(kernel: str) -> str:
    """sha256 (16 hex digits) of the sources `kernel` is compiled from: its .hip file and
    every header it includes from csrc/ or include/, transitively."""
    import re
    csrc = os.path.join(ROOT, "long_context_sparse_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    seen, todo = [], [KERNEL_SOURCE[kernel]]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        path = next((os.path.join(d, name) for d in (csrc, inc) if os.path.exists(os.path.join(d, name))), None)
        if path is None:
            continue
        seen.append(name)
        todo += re.findall(r'^\s*#include\s+"([^"]+)"', open(path).read(), flags=re.M)
    h = hashlib.sha256()
    for name in sorted(seen):
        path = next(os.path.join(d, name) for d in (csrc, inc) if os.path.exists(os.path.join(d, name)))
        with open(path, "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(label: str, kernel: str) -> str:
    """File name of the counter summary of `kernel` on workload `label` ("@" -> "_")."""
    return f"{kernel}_{label.replace('@', '_')}_traffic.md"


def read_traffic(workload: str, kernel: str) -> Optional[float]:
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", traffic_file(workload, KERNEL_NAMES.get(kernel, kernel)))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_sources_sha256") != kernel_source_hash(KERNEL_NAMES.get(kernel, kernel)):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ GPU measurement
_SLEEP_CYCLES_PER_US: List[float] = []


def gpu_wait(us: float) -> None:
    """Occupies the current stream for about `us` microseconds (torch's spin kernel,
    calibrated once), so that launches enqueued behind it start back to back."""
    import torch
    if not _SLEEP_CYCLES_PER_US:
        torch.cuda._sleep(1000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US.append(1_000_000 / max(a.elapsed_time(b) * 1e3, 1.0))
    torch.cuda._sleep(int(us * _SLEEP_CYCLES_PER_US[0]))


def measure(label: str, steps: int, warmup: int, cold_iters: int, calib_copy: bool, minimal: bool = False) -> Dict:
    """One workload; label = a workload name, optionally with "@topkK" (static top-k rule,
    budget K tokens).  minimal: only the warm-up, the timed steps and the per-launch timing
    (for profiler runs whose traces should hold the step's kernels alone)."""
    import torch

    import workloads as W
    from long_context_sparse_amd import DecodeStep, StepShape

    name, _, rule = label.partition("@")
    k_tokens = int(rule[4:]) if rule.startswith("topk") else 0
    if rule and not k_tokens:
        raise ValueError(f"unknown selection rule in {label!r}")
    cfg = W.get_config(name)
    t0 = time.time()
    inp = W.make_inputs(cfg)
    log(f"[bench] {label}: inputs built in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    t = W.to_device(inp, dev)
    shape = StepShape(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, n_ret=cfg.n_ret, n_loc=cfg.n_loc, max_ctx=cfg.max_ctx,
                      block=cfg.block, split_tokens=cfg.split_tokens, window=cfg.window, sinks=cfg.sinks)
    step = DecodeStep(shape, device=dev, k_tokens=k_tokens)
    step(t)
    torch.cuda.synchronize()
    sel_idx = step.sel_idx.cpu().numpy()
    sel_cnt = step.sel_cnt.cpu().numpy()
    alg = algorithmic_bytes(cfg, inp, sel_idx, sel_cnt)
    if k_tokens:
        alg["index_topk"] = alg.pop("index_topp")

    # timed region: `steps` back-to-back decode steps, inputs resident in HBM, between two
    # events on the stream they run on.  The steps are queued behind a spin of ~60 us a
    # step, so the GPU runs them back to back: the events time the GPU's work, and a host
    # stall while queueing (or a host slower than the step) does not show up as GPU idle
    # time; the host's own queueing rate is reported beside it.  The per-step spread comes
    # from a second block of `steps` steps with an event after every step: each such event
    # is a marker packet of its own on the stream (2.5-5 us a step measured), so that block
    # times the steps plus their markers and gives the distribution, not the mean.
    main = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        step(t)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_wait(60.0 * steps)
    w0 = time.perf_counter()
    ev0.record(main)
    for i in range(steps):
        step(t)
    ev1.record(main)
    wall = time.perf_counter() - w0
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / steps
    evs_step = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    gpu_wait(60.0 * steps)
    evs_step[0].record(main)
    for i in range(steps):
        step(t)
        evs_step[i + 1].record(main)
    torch.cuda.synchronize()
    per_step_us = [evs_step[i].elapsed_time(evs_step[i + 1]) * 1e3 for i in range(steps)]
    log(f"[bench] {label}: {steps} steps, {ms_per_step * 1e3:.1f} us/step (per-step events: median "
        f"{np.median(per_step_us):.1f}; host queueing {wall * 1e6 / steps:.1f} us/step)")
    # per-launch durations: each of the step's three launches repeated back to back on the
    # stream the step runs on (every launch rewrites the same outputs from the same
    # inputs), one event pair around each block of `reps` launches, the median of three
    # blocks.  A block is queued behind a GPU-side wait long enough for the host to
    # enqueue all of it, so the GPU runs the launches back to back whatever the host's
    # per-call cost.
    calls = [("index_topk", step.index_topk) if k_tokens else ("index_topp", step.index_topp),
             ("decode_attn", step.attn), ("decode_merge", step.merge)]
    if not cfg.n_ret:
        calls = calls[1:]
    reps = 20
    kern_us = {}
    for k, f in calls:
        f(t, main)
        blocks = []
        for _ in range(3):  # the median of three blocks (a host stall longer than the wait shows in one)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            gpu_wait(reps * 100.0)
            e0.record(main)
            for _ in range(reps):
                f(t, main)
            e1.record(main)
            torch.cuda.synchronize()
            blocks.append(e0.elapsed_time(e1) * 1e3 / reps)
        kern_us[k] = float(np.median(blocks))
    if calib_copy:
        # plain device copy of known size, for scaling HBM counters (1 GiB read + 1 GiB written)
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if minimal:
        res = dict(workload=name, label=label, k_tokens=k_tokens, cfg=cfg, inp=inp, alg=alg, latency_us=ms_per_step * 1e3,
                   per_step_us=per_step_us, wall_us=wall * 1e6 / steps, kern_us=kern_us,
                   dominant=max(kern_us, key=kern_us.get), append_us=None, cold_us=None, dense_us=None,
                   gbs=alg["step"] / (ms_per_step * 1e-3) / 1e9, sel_frac=None)
        del step, t
        torch.cuda.empty_cache()
        return res

    # cold caches: a 1 GiB write evicts L2 and the 256 MB last-level cache before each step
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(cold_iters):
        flush.fill_(1.0)
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(main)
        step(t)
        b_.record(main)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b_) * 1e3)
    del flush

    # the decode-side cache append before the step (not part of the step): the last
    # token's K/V rows and index keys rewritten from the token itself
    from long_context_sparse_amd import abi
    lens = [int(n) for n in inp.seq_lens]
    k_new = torch.stack([t["k_cache"][b, :, n - 1] for b, n in enumerate(lens)]).contiguous()
    v_new = torch.stack([t["v_cache"][b, :, n - 1] for b, n in enumerate(lens)]).contiguous()
    w_k = torch.from_numpy(np.ascontiguousarray(inp.w_k)).view(torch.bfloat16).to(dev) if cfg.n_ret else None
    append = lambda: abi.rtp_cache_append(k_new, v_new, k_new, w_k, t["seq_lens"], t["ret_heads"], cfg.B,  # noqa
                                          cfg.Hq, cfg.Hkv, cfg.n_ret, cfg.max_ctx, t["k_cache"], t["v_cache"],
                                          t["k_idx"], main, sinks=cfg.sinks, window=cfg.window,
                                          **DecodeStep.placement(t))
    for _ in range(5):
        append()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(main)
    for _ in range(50):
        append()
    a1.record(main)
    torch.cuda.synchronize()
    append_us = a0.elapsed_time(a1) * 1e3 / 50

    # context: dense decode of every query head over every cached token, on the same
    # attention core (the local heads' call with the window covering the context, no
    # sinks); the sparse step's speedup over it stands beside the pages' speedup over
    # FlashAttention-2 (other hardware)
    all_heads = torch.arange(cfg.Hq, dtype=torch.int32, device=dev)
    ws_d = torch.zeros(abi.rtp_local_window_workspace_size(cfg.B, cfg.Hq, cfg.Hkv, cfg.Hq, cfg.max_ctx, cfg.max_ctx, 0),
                       dtype=torch.uint8, device=dev)
    out_d = torch.empty((cfg.B, cfg.Hq, 128), dtype=torch.float32, device=dev)
    dense = lambda: abi.rtp_local_window_attn(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], all_heads,  # noqa
                                              cfg.B, cfg.Hq, cfg.Hkv, cfg.Hq, cfg.max_ctx, cfg.max_ctx, 0, out_d,
                                              ws_d, main)
    dense()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(main)
    for _ in range(10):
        dense()
    d1.record(main)
    torch.cuda.synchronize()
    dense_us = d0.elapsed_time(d1) * 1e3 / 10
    del ws_d, out_d

    lat_us = ms_per_step * 1e3
    dom = max(kern_us, key=kern_us.get)
    res = dict(
        workload=name, label=label, k_tokens=k_tokens, cfg=cfg, inp=inp, alg=alg, latency_us=lat_us,
        per_step_us=per_step_us, wall_us=wall * 1e6 / steps,
        kern_us=kern_us, dominant=dom, append_us=append_us, cold_us=float(np.median(cold)) if cold else None,
        dense_us=dense_us,
        gbs=alg["step"] / (lat_us * 1e-6) / 1e9,
        sel_frac=float(np.mean([sel_cnt[b, r] / -(-int(inp.seq_lens[b]) // cfg.block)
                                for b in range(cfg.B) for r in range(cfg.n_ret)])) if cfg.n_ret else 0.0,
    )
    del step, t
    torch.cuda.empty_cache()
    return res


PEAK_MFMA_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA, vendor figure


def prefill_flops(N: int, n_ret: int, n_loc: int, window: int, sinks: int) -> float:
    """Algorithmic flops of one prefill pass: 4 x 128 per attended (query, key) pair (the
    q.k dot product and the p.v update).  Position i attends to i + 1 keys in a
    retrieval head and to min(i + 1, S + W) in a local head (sinks + window)."""
    dense = N * (N + 1) // 2
    cap = sinks + window
    local = (min(N, cap) * (min(N, cap) + 1) // 2) + max(0, N - cap) * cap
    return 4.0 * 128 * (n_ret * dense + n_loc * local)


def measure_prefill(N: int, reps: int, dense_too: bool) -> Dict:
    """rtp_prefill_attn over one N-token prompt at the pages' prefill configuration
    (32 query heads on 8 KV heads, 5 retrieval heads ~ 15%, sink 4 + window 8192);
    synthetic N(0, 1) rows drawn on the device from a fixed seed."""
    import torch

    from long_context_sparse_amd import abi

    Hq, Hkv, W_, S_ = 32, 8, 8192, 4
    ret = [3, 9, 15, 20, 30]
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(N)
    q = torch.randn((1, Hq, N, 128), generator=gen, device=dev).to(torch.bfloat16)
    k = torch.randn((1, Hkv, N, 128), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((1, Hkv, N, 128), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((1, Hq, N, 128), dtype=torch.float32, device=dev)
    lens = torch.tensor([N], dtype=torch.int32, device=dev)

    def run(heads):
        rh = torch.tensor(heads, dtype=torch.int32, device=dev)
        call = lambda: abi.rtp_prefill_attn(q, k, v, lens, rh, 1, Hq, Hkv, len(heads), N, W_, S_, out)  # noqa
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms = run(ret)
    # the prompt's index keys for the retrieval heads (rtp_prefill_index_keys)
    w_k = torch.randn((len(ret), 16, 128), generator=gen, device=dev).to(torch.bfloat16)
    k_idx = torch.empty((1, len(ret), N, 16), dtype=torch.bfloat16, device=dev)
    rh = torch.tensor(ret, dtype=torch.int32, device=dev)
    keys = lambda: abi.rtp_prefill_index_keys(k, w_k, lens, rh, 1, Hq, Hkv, len(ret), N, k_idx)  # noqa
    keys()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        keys()
    e1.record()
    torch.cuda.synchronize()
    keys_ms = e0.elapsed_time(e1) / reps
    fl = prefill_flops(N, len(ret), Hq - len(ret), W_, S_)
    tf = fl / (ms * 1e-3) / 1e12
    res = {"latency_ms": round(ms, 3), "tflops": round(tf, 1), "index_keys_ms": round(keys_ms, 3),
           "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tf, 1),
                        "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_TFLOPS, 4),
                        "traffic": read_traffic(f"prefill{N // 1024}k", "prefill_kernel"),
                        "alg_flops_per_launch": fl, "avg_launch_us": round(ms * 1e3, 1)},
           "config": {"workload": f"prefill{N // 1024}k", "batch": 1, "ctx": N, "kv_heads": Hkv, "q_heads": Hq,
                      "retrieval_heads": len(ret), "head_dim": 128, "window": W_, "sinks": S_}}
    log(f"[bench] prefill {N}: {ms:.3f} ms, {tf:.1f} TFLOP/s; prompt index keys {keys_ms:.3f} ms")
    if dense_too:
        dms = run(list(range(Hq)))
        dfl = prefill_flops(N, Hq, 0, W_, S_)
        res["dense_causal_ms"] = round(dms, 3)
        res["dense_causal_tflops"] = round(dfl / (dms * 1e-3) / 1e12, 1)
        res["speedup_vs_dense"] = round(dms / ms, 2)
        log(f"[bench] prefill {N} all heads dense: {dms:.3f} ms ({dms / ms:.2f}x the sparse pass)")
    del q, k, v, out, k_idx
    torch.cuda.empty_cache()
    return res


def config_of(cfg, k_tokens: int = 0) -> Dict:
    ctx = sorted(set(cfg.ctx))
    sel = {"top_k_tokens": k_tokens} if k_tokens else {"top_p": sorted(set(cfg.top_p))}
    return {"workload": cfg.name, "batch": cfg.B, "ctx": ctx[0] if len(ctx) == 1 else [min(ctx), max(ctx)],
            "kv_heads": cfg.Hkv, "q_heads": cfg.Hq, "retrieval_heads": cfg.n_ret, "head_dim": 128,
            "index_dim": 16, "block": cfg.block, **sel, "window": cfg.window,
            "sinks": cfg.sinks, "split_tokens": cfg.split_tokens}


def roofline_of(r: Dict) -> Dict:
    k = r["dominant"]
    us = r["kern_us"][k]
    ach = r["alg"][k] / (us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": KERNEL_NAMES[k], "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(r["label"], k),
            "alg_bytes_per_launch": int(r["alg"][k]), "avg_launch_us": round(us, 2)}


# ------------------------------------------------------------------ CPU baseline
_ORACLE_ARRAYS = ("seq_lens", "ret_heads", "loc_heads", "top_p", "q", "w_q", "k_cache", "v_cache", "k_idx")


def _oracle_worker(args):
    """Pool worker (a fresh interpreter that never touches the GPU): the oracle on a share
    of the step's (sequence, head) items, reading the inputs from shared memory."""
    import types
    from multiprocessing import shared_memory

    from oracle import rtp_oracle as O
    cfg, specs, items = args
    shms, arrs = [], {}
    for name, (shm_name, shape, dtype) in specs.items():
        shm = shared_memory.SharedMemory(name=shm_name)
        shms.append(shm)
        arrs[name] = np.ndarray(shape, dtype=dtype, buffer=shm.buf)
    inp = types.SimpleNamespace(cfg=cfg, q_pre=arrs["q"], **arrs)
    t0 = time.perf_counter()
    O.decode_step(inp, items)
    dt = time.perf_counter() - t0
    del inp, arrs
    for shm in shms:
        shm.close()
    return dt


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(r: Dict, reps: int) -> Dict:
    """The fp64 oracle (unchanged) over the whole step of the same workload on the host:
    once on one core (one BLAS thread), once on every core this process may use (a pool of
    fresh worker processes over the step's (sequence, head) items, inputs in shared
    memory, one BLAS thread each); median of `reps` runs each."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    from threadpoolctl import threadpool_limits

    from oracle import rtp_oracle as O

    inp, cfg = r["inp"], r["cfg"]
    one = []
    with threadpool_limits(limits=1):
        for _ in range(reps):
            t0 = time.perf_counter()
            O.decode_step(inp)
            one.append(time.perf_counter() - t0)
    sec1 = statistics.median(one)

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    items = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    shms, specs = [], {}
    try:
        for name in _ORACLE_ARRAYS:
            a = np.ascontiguousarray(getattr(inp, name))
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            shms.append(shm)
            specs[name] = (shm.name, a.shape, a.dtype.str)
        # the heaviest items first, dealt round-robin, so the shares finish together
        shares = [items[i::cores] for i in range(cores)]
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"
        try:
            ctx = mp.get_context("spawn")
            with ctx.Pool(cores) as pool:
                pool.map(_oracle_worker, [(cfg, specs, sh[:1]) for sh in shares])  # workers warm
                multi = []
                for _ in range(reps):
                    t0 = time.perf_counter()
                    pool.map(_oracle_worker, [(cfg, specs, sh) for sh in shares])
                    multi.append(time.perf_counter() - t0)
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    secn = statistics.median(multi)
    gb = r["alg"]["step"] / 1e9
    return {"value": round(gb / secn, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole {cfg.name} step ({cfg.B} seqs x {cfg.Hq} heads, every head), median of {reps} runs "
                      f"on {cores} cores ({secn:.3f} s) and on 1 core ({sec1:.3f} s); GB/s = the step's "
                      f"algorithmic bytes / oracle time",
            "seconds_per_step": round(secn, 4), "one_core": {"value": round(gb / sec1, 4), "seconds_per_step":
                                                              round(sec1, 4), "cores": 1},
            "cpu_model": cpu_model()}


# ------------------------------------------------------------------ streaming ceiling
def stream_ceiling(gib: float = 4.0, reps: int = 10) -> Dict:
    """A plain read-only stream (rtp_stream_read) over a fresh `gib` GiB buffer, with
    non-temporal and with cached 16-byte loads, at a few grid sizes; the best of each."""
    import torch

    from long_context_sparse_amd import abi

    nbytes = int(gib * (1 << 30))
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(65535, dtype=torch.int32, device="cuda")
    out = {}
    for nt in (True, False):
        best = 0.0
        for wgs in (1024, 2048, 4096, 8192):
            abi.rtp_stream_read(buf, sink, wgs, nt)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                abi.rtp_stream_read(buf, sink, wgs, nt)
            e1.record()
            torch.cuda.synchronize()
            gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
            best = max(best, gbs)
        out["nontemporal_gbs" if nt else "cached_gbs"] = round(best, 1)
    del buf, sink
    torch.cuda.empty_cache()
    out["bytes"] = nbytes
    log(f"[bench] streaming read ceiling: {out['nontemporal_gbs']} GB/s non-temporal, {out['cached_gbs']} GB/s cached")
    return out


def mfma_ceiling(iters: int = 4096, reps: int = 5) -> Dict:
    """Back-to-back bf16 32x32x16 MFMAs on every SIMD (rtp_mfma_rate) at a few grid sizes,
    the best TFLOP/s: with seeded N(0, 1) operands (like the prefill's q and K), the
    ceiling the MFMA-bound prefill is compared with, and with all-one operands, which the
    part runs at a higher clock."""
    import torch

    from long_context_sparse_amd import abi

    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    operands = {"normal": torch.randn((2, 64, 8), generator=g, device="cuda").to(torch.bfloat16),
                "ones": torch.ones((2, 64, 8), device="cuda", dtype=torch.bfloat16)}
    res = {}
    for kind, ops in operands.items():
        best = 0.0
        for wgs in (1024, 2048, 4096):
            out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
            abi.rtp_mfma_rate(ops, out, wgs, iters)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                abi.rtp_mfma_rate(ops, out, wgs, iters)
            e1.record()
            torch.cuda.synchronize()
            flops = wgs * 16.0 * iters * 32768.0 * reps
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
            del out
        res["bf16_tflops" if kind == "normal" else "bf16_tflops_all_one_operands"] = round(best, 1)
    res["frac_of_rated_peak"] = round(res["bf16_tflops"] / PEAK_MFMA_TFLOPS, 4)
    log(f"[bench] MFMA ceiling: {res['bf16_tflops']} TFLOP/s bf16 with N(0,1) operands "
        f"({res['frac_of_rated_peak']} of the rated {PEAK_MFMA_TFLOPS:.0f}); "
        f"{res['bf16_tflops_all_one_operands']} with all-one operands")
    return res


def step_stats(r: Dict) -> Dict:
    """Median, 10th and 90th percentile of the per-step durations (µs) and their GB/s,
    from the block timed with an event after every step (each step's time includes its
    event's marker packet; the mean latency comes from the block without them)."""
    v = np.asarray(r["per_step_us"], dtype=np.float64)
    p10, p50, p90 = (float(np.percentile(v, q)) for q in (10, 50, 90))
    gb = r["alg"]["step"] / 1e3
    return {"median_us": round(p50, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
            "median_effective_gbs": round(gb / p50, 1), "steps": int(v.size), "includes_step_events": True}


def main(argv: Optional[List[str]] = None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ctx128k")
    ap.add_argument("--also", default="ctx1m,ctx128k@topk4096,mixed,ctx32k,tiny",
                    help="comma-separated extra workloads ('' for none); name@topkK: static top-k rule")
    ap.add_argument("--prefill", default="32768,131072",
                    help="comma-separated prompt lengths for the prefill pass ('' for none)")
    ap.add_argument("--cold-iters", type=int, default=20)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true", help="skip the measured HBM and MFMA ceilings")
    ap.add_argument("--minimal", action="store_true",
                    help="per workload only the warm-up, the timed steps and the per-launch timing, and the "
                         "prefill passes asked for (for profiler runs)")
    ap.add_argument("--calib-copy", action="store_true", help="also run a 1 GiB device copy (counter scaling)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); the path shards by sequence, "
              "KV head or context across GPUs, which is not implemented here.", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    head = measure(a.workload, a.steps, a.warmup, a.cold_iters, a.calib_copy, a.minimal)
    extras = {}
    for name in [x for x in a.also.split(",") if x and x != a.workload]:
        extras[name] = measure(name, a.steps, a.warmup, a.cold_iters, False, a.minimal)
    prefill = {}
    for n in [int(x) for x in a.prefill.split(",") if x]:
        prefill[f"prefill{n // 1024}k"] = measure_prefill(n, 5 if n <= 65536 else 2, dense_too=n <= 131072)
    if a.minimal:
        print(json.dumps({"minimal": True, **{r["label"]: {
            "latency_us": round(r["latency_us"], 2), "per_step": step_stats(r),
            "call_us": {CALL_NAMES[k]: round(v, 2) for k, v in r["kern_us"].items()},
            "alg_bytes": {CALL_NAMES[k]: int(r["alg"][k]) for k in r["kern_us"]},
            "roofline": roofline_of(r)} for r in [head, *extras.values()]}, "prefill": prefill}), flush=True)
        return 0

    ceiling = None if a.no_stream_ceiling else stream_ceiling()
    mceil = None if a.no_stream_ceiling or not prefill else mfma_ceiling()
    if mceil:
        for v in prefill.values():
            v["roofline"]["frac_of_measured_mfma_ceiling"] = round(v["roofline"]["achieved"] / mceil["bf16_tflops"], 4)

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(head, a.cpu_reps)

    def roof(r):
        x = roofline_of(r)
        if ceiling:
            x["frac_of_measured_stream_ceiling"] = round(x["achieved"] / ceiling["nontemporal_gbs"], 4)
        return x

    def summary(r):
        return {"latency_us": round(r["latency_us"], 2), "effective_gbs": round(r["gbs"], 1),
                "frac_of_peak": round(r["gbs"] / PEAK_HBM_GBS, 4), "alg_bytes": int(r["alg"]["step"]),
                "per_step": step_stats(r),
                "host_queueing_us_per_step": round(r["wall_us"], 2),
                "cold_latency_us": None if r["cold_us"] is None else round(r["cold_us"], 2),
                "cold_effective_gbs": None if not r["cold_us"] else round(r["alg"]["step"] / r["cold_us"] / 1e3, 1),
                "call_us": {CALL_NAMES[k]: round(v, 2) for k, v in r["kern_us"].items()},
                "cache_append_us": round(r["append_us"], 2),
                "dense_decode_us": round(r["dense_us"], 1),
                "speedup_vs_dense_decode": round(r["dense_us"] / r["latency_us"], 2),
                "mean_selected_block_fraction": round(r["sel_frac"], 4),
                "roofline": roof(r), "config": config_of(r["cfg"], r["k_tokens"])}

    line = {
        "metric": METRIC, "value": round(head["gbs"], 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(head["latency_us"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": config_of(head["cfg"], head["k_tokens"]),
        "latency_us": round(head["latency_us"], 2),
        "frac_of_peak": round(head["gbs"] / PEAK_HBM_GBS, 4),
        "per_step": step_stats(head),
        "roofline": roof(head),
        "cpu_baseline": cpu,
        "stream_ceiling": ceiling,
        "mfma_ceiling": mceil,
        "detail": summary(head),
        "also": {k: summary(v) for k, v in extras.items()},
        "prefill": prefill,
        # the pages' own speedups over FlashAttention-2, quoted for context only (their
        # hardware, their baseline); the lines above carry this path's dense ratios
        "pages_context": {"decode_speedup_vs_fa2": "1.47x at 32K to 2.01x at 1M",
                          "prefill_speedup_vs_fa2": "2.83x at 32K to 9.36x at 1M", "hardware": "NVIDIA H20"},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
