"""Seeded synthetic decode workloads for RTPurbo-style sparse decode attention.

This module only *builds inputs*: bf16 caches, queries, projection matrices,
head lists, per-head top-p values and sequence lengths, drawn from seeded
counter-style streams so that every (tensor, sequence, head) can be rebuilt on
its own.  It holds none of the path's arithmetic (no softmax, no selection, no
attention).  The one projection it evaluates, ``W^Q q``, is used only to aim
planted "needle" index keys at a head's index query; consumers recompute
everything they need from the returned arrays.

Both the CPU oracle and the GPU path consume the arrays returned by
:func:`make_inputs`; neither imports the other.

All bf16 tensors are returned as ``numpy.uint16`` bit patterns
(round-to-nearest-even from float32, or directly from float64 for values built
in float64).

The five named workloads restate the decode configurations the method is
measured on (RTPurbo, "Full Attention Strikes Back", efficiency section: 32K to
1M context; main configuration r=16, sink 4, window 8192, top-p 0.9,
retrieval-head ratio about 15%).  Benchmark suites used on the pages (RULER,
LongBench) and trained projections are not available; the peaked / diffuse
query mix below stands in for single-needle vs multi-key retrieval.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

HEAD_DIM = 128
INDEX_DIM = 16

# tensor ids for the seed streams
_T_Q, _T_WQ, _T_WK, _T_K, _T_V, _T_HEADS, _T_LENS, _T_PLANT, _T_P, _T_KIND = range(1, 11)
_T_PQ = 11          # prefill queries (one per prompt position)


# --------------------------------------------------------------------------- bf16
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 straight to bf16 (nearest-even, normal range only)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    drop = np.uint64(45)  # 52 mantissa bits -> 7
    half = np.uint64((1 << 44) - 1)
    r = (u + half + ((u >> drop) & np.uint64(1))) & ~np.uint64((1 << 45) - 1)
    y = r.view(np.float64).astype(np.float32)  # exact: <= 8 significant bits
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


# ------------------------------------------------------------------------- configs
@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One decode-step workload.

    ``kind`` selects how index keys are planted:
      * ``needles3x``      needle blocks whose index keys are 3x the head's index query
      * ``peaked_diffuse`` half the (sequence, retrieval head) pairs get one needle
                           block at score margin +6, the other half are flattened by
                           0.25 with 10% of blocks boosted by +2
      * ``depth_needles``  needles at context depths 0.1 / 0.5 / 0.9, margin +6
      * ``random``         no planting
      * ``flat``           every index key equal (all full blocks tie exactly)
      * ``near_flat``      index scores spread by about 1e-3 (near ties)
    """

    name: str
    seed: int
    B: int
    Hkv: int
    Hq: int
    n_ret: int
    ctx: Tuple[int, ...]            # per-sequence context lengths N_b (incl. current token)
    block: int
    top_p: Tuple[float, ...]        # per retrieval head (shared by the batch)
    window: int
    sinks: int
    split_tokens: int
    kind: str = "random"
    needles: Tuple[int, int] = (2, 2)   # needles3x: inclusive range of needle count per (b, r)
    shared_needles: bool = False        # needles3x: same needle blocks for every head
    plant_full_key: bool = False        # needles3x: also plant full K = 3 q of the group's first head
    ret_heads: Optional[Tuple[int, ...]] = None  # explicit retrieval head ids (else seeded choice)

    @property
    def max_ctx(self) -> int:
        return int(max(self.ctx))

    @property
    def n_loc(self) -> int:
        return self.Hq - self.n_ret

    @property
    def gqa(self) -> int:
        return self.Hq // self.Hkv


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _mixed_ctx(seed: int) -> Tuple[int, ...]:
    g = _rng(seed, _T_LENS)
    return tuple(int(v) for v in g.integers(8192, 262144, size=16, endpoint=True))


def _mixed_p(seed: int, n_ret: int) -> Tuple[float, ...]:
    g = _rng(seed, _T_P)
    return tuple(float(v) for v in g.choice(np.array([0.9, 0.95, 0.99]), size=n_ret))


def _named() -> Dict[str, DecodeConfig]:
    c = {}
    c["tiny"] = DecodeConfig(
        name="tiny", seed=1, B=1, Hkv=1, Hq=4, n_ret=4, ctx=(4096,), block=64,
        top_p=(0.9,) * 4, window=0, sinks=0, split_tokens=1024, kind="needles3x",
        needles=(2, 2), shared_needles=True, plant_full_key=True,
        ret_heads=(0, 1, 2, 3))
    c["ctx32k"] = DecodeConfig(
        name="ctx32k", seed=2, B=1, Hkv=8, Hq=32, n_ret=8, ctx=(32768,), block=64,
        top_p=(0.95,) * 8, window=1024, sinks=4, split_tokens=2048, kind="needles3x",
        needles=(1, 8))
    # window unspecified for 128K and 1M: the pages' main configuration (8192 + 4 sinks)
    c["ctx128k"] = DecodeConfig(
        name="ctx128k", seed=3, B=4, Hkv=8, Hq=32, n_ret=8, ctx=(131072,) * 4, block=64,
        top_p=(0.95,) * 8, window=8192, sinks=4, split_tokens=1024, kind="peaked_diffuse")
    c["ctx1m"] = DecodeConfig(
        name="ctx1m", seed=4, B=1, Hkv=8, Hq=32, n_ret=4, ctx=(1 << 20,), block=128,
        top_p=(0.95,) * 4, window=8192, sinks=4, split_tokens=65536, kind="depth_needles")
    c["mixed"] = DecodeConfig(
        name="mixed", seed=5, B=16, Hkv=8, Hq=32, n_ret=6, ctx=_mixed_ctx(5), block=64,
        top_p=_mixed_p(5, 6), window=2048, sinks=4, split_tokens=4096, kind="peaked_diffuse")
    return c


CONFIGS: Dict[str, DecodeConfig] = _named()


def get_config(name: str) -> DecodeConfig:
    return CONFIGS[name]


# -------------------------------------------------------------------------- inputs
@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    seq_lens: np.ndarray      # int32 [B]
    ret_heads: np.ndarray     # int32 [n_ret], ascending query-head ids
    loc_heads: np.ndarray     # int32 [n_loc], ascending query-head ids
    top_p: np.ndarray         # float32 [B, n_ret]
    q: np.ndarray             # bf16 bits [B, Hq, 128]  (query; no RoPE here, so also q_pre)
    w_q: np.ndarray           # bf16 bits [n_ret, 16, 128]
    w_k: np.ndarray           # bf16 bits [n_ret, 16, 128]
    k_cache: np.ndarray       # bf16 bits [B, Hkv, max_ctx, 128]
    v_cache: np.ndarray       # bf16 bits [B, Hkv, max_ctx, 128]
    k_idx: np.ndarray         # bf16 bits [B, n_ret, max_ctx, 16]
    needles: Dict[Tuple[int, int], List[int]]
    peaked: Dict[Tuple[int, int], bool]

    @property
    def q_pre(self) -> np.ndarray:
        return self.q


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_normal(dst: np.ndarray, key: Tuple[int, ...], n_rows: int, row: int) -> None:
    g = _rng(*key)
    dst[:n_rows] = f32_to_bf16_bits(g.standard_normal(n_rows * row, dtype=np.float32)).reshape(n_rows, row)


def _index_query_f64(w_q_r: np.ndarray, q_row: np.ndarray) -> np.ndarray:
    # used only to aim planted index keys
    return bf16_bits_to_f32(w_q_r).astype(np.float64) @ bf16_bits_to_f32(q_row).astype(np.float64)


def make_inputs(cfg: DecodeConfig, seed: Optional[int] = None, pad_value: int = 0,
                workers: Optional[int] = None) -> DecodeInputs:
    """Build the seeded inputs of one decode step for ``cfg``.

    ``pad_value`` (bf16 bits) fills cache rows at or beyond each sequence's
    length; pass ``BF16_NAN`` to poison them.
    """
    s = cfg.seed if seed is None else seed
    B, Hkv, Hq, R, Tm = cfg.B, cfg.Hkv, cfg.Hq, cfg.n_ret, cfg.max_ctx
    assert Hq % Hkv == 0 and 0 <= R <= Hq and len(cfg.ctx) == B
    assert all(1 <= n for n in cfg.ctx) and len(cfg.top_p) == R
    G = Hq // Hkv
    seq_lens = np.asarray(cfg.ctx, dtype=np.int32)

    if cfg.ret_heads is not None:
        ret = np.asarray(sorted(cfg.ret_heads), dtype=np.int32)
    else:
        ret = np.sort(_rng(s, _T_HEADS).choice(Hq, size=R, replace=False)).astype(np.int32)
    assert len(ret) == R
    loc = np.asarray([h for h in range(Hq) if h not in set(ret.tolist())], dtype=np.int32)
    top_p = np.tile(np.asarray(cfg.top_p, dtype=np.float32)[None, :], (B, 1))

    g = _rng(s, _T_Q)
    q = f32_to_bf16_bits(g.standard_normal(B * Hq * HEAD_DIM, dtype=np.float32)).reshape(B, Hq, HEAD_DIM)
    wscale = np.float32(1.0 / np.sqrt(HEAD_DIM))
    w_q = np.empty((R, INDEX_DIM, HEAD_DIM), np.uint16)
    w_k = np.empty((R, INDEX_DIM, HEAD_DIM), np.uint16)
    for r in range(R):
        w_q[r] = f32_to_bf16_bits(_rng(s, _T_WQ, r).standard_normal((INDEX_DIM, HEAD_DIM), dtype=np.float32) * wscale)
        w_k[r] = f32_to_bf16_bits(_rng(s, _T_WK, r).standard_normal((INDEX_DIM, HEAD_DIM), dtype=np.float32) * wscale)

    k_cache = np.full((B, Hkv, Tm, HEAD_DIM), pad_value, np.uint16)
    v_cache = np.full((B, Hkv, Tm, HEAD_DIM), pad_value, np.uint16)
    jobs = []
    for b in range(B):
        n = int(seq_lens[b])
        for kv in range(Hkv):
            jobs.append((k_cache[b, kv], (s, _T_K, b, kv), n))
            jobs.append((v_cache[b, kv], (s, _T_V, b, kv), n))
    nw = workers or _workers()
    with ThreadPoolExecutor(nw) as ex:
        list(ex.map(lambda a: _fill_normal(a[0], a[1], a[2], HEAD_DIM), jobs))

    needles: Dict[Tuple[int, int], List[int]] = {}
    peaked: Dict[Tuple[int, int], bool] = {}
    k_idx = np.full((B, R, Tm, INDEX_DIM), pad_value, np.uint16)

    pairs = [(b, r) for b in range(B) for r in range(R)]
    if cfg.kind == "peaked_diffuse":
        perm = _rng(s, _T_KIND).permutation(len(pairs))
        for i, pi in enumerate(perm):
            peaked[pairs[pi]] = i < (len(pairs) + 1) // 2

    def build_head(br: Tuple[int, int]) -> None:
        b, r = br
        n = int(seq_lens[b])
        nblk = -(-n // cfg.block)
        kv = int(ret[r]) // G
        wk = bf16_bits_to_f32(w_k[r]).astype(np.float64)          # [16, 128]
        raw = np.empty((n, INDEX_DIM), np.float64)
        step = 1 << 15
        for t0 in range(0, n, step):
            t1 = min(n, t0 + step)
            raw[t0:t1] = bf16_bits_to_f32(k_cache[b, kv, t0:t1]).astype(np.float64) @ wk.T
        qi = _index_query_f64(w_q[r], q[b, int(ret[r])])
        qn = qi / float(qi @ qi)                       # unit index score along q_idx
        gp = _rng(s, _T_PLANT, b, r)
        blocks: List[int] = []
        if cfg.kind == "needles3x":
            if cfg.shared_needles:
                gs = _rng(s, _T_PLANT, b)
                cnt = int(gs.integers(cfg.needles[0], cfg.needles[1], endpoint=True))
                blocks = sorted(int(x) for x in gs.choice(nblk, size=min(cnt, nblk), replace=False))
            else:
                cnt = int(gp.integers(cfg.needles[0], cfg.needles[1], endpoint=True))
                blocks = sorted(int(x) for x in gp.choice(nblk, size=min(cnt, nblk), replace=False))
            kb = f64_to_bf16_bits(raw)
            kn = f64_to_bf16_bits(3.0 * qi)
            for j in blocks:
                kb[j * cfg.block:min(n, (j + 1) * cfg.block)] = kn
        elif cfg.kind == "depth_needles" or (cfg.kind == "peaked_diffuse" and peaked[(b, r)]):
            if cfg.kind == "depth_needles":
                blocks = sorted({int(np.floor(d * n)) // cfg.block for d in (0.1, 0.5, 0.9)})
            else:
                blocks = [int(gp.integers(0, nblk))]
            kb = f64_to_bf16_bits(raw)
            mask = np.ones(n, bool)
            for j in blocks:
                mask[j * cfg.block:min(n, (j + 1) * cfg.block)] = False
            s_bg = bf16_bits_to_f32(kb[mask]).astype(np.float64) @ qi if mask.any() else np.zeros(1)
            target = float(s_bg.max()) + 6.0
            kn = f64_to_bf16_bits(target * qn)
            for j in blocks:
                kb[j * cfg.block:min(n, (j + 1) * cfg.block)] = kn
        elif cfg.kind == "peaked_diffuse":
            flat = 0.25 * raw
            nboost = max(1, int(round(0.1 * nblk)))
            blocks = sorted(int(x) for x in gp.choice(nblk, size=nboost, replace=False))
            for j in blocks:
                flat[j * cfg.block:min(n, (j + 1) * cfg.block)] += 2.0 * qn
            kb = f64_to_bf16_bits(flat)
        elif cfg.kind == "random":
            kb = f64_to_bf16_bits(raw)
        elif cfg.kind == "flat":
            # every index key equal: every full block has the same mass (exact ties)
            kb = np.tile(f64_to_bf16_bits(0.5 * qn), (n, 1))
        elif cfg.kind == "near_flat":
            # scores spread by about 1e-3: many blocks within a tiny mass range
            kb = f64_to_bf16_bits(1e-3 * raw + 0.5 * qn)
        else:
            raise ValueError(f"unknown workload kind {cfg.kind!r}")
        k_idx[b, r, :n] = kb
        needles[(b, r)] = blocks

    with ThreadPoolExecutor(nw) as ex:
        list(ex.map(build_head, pairs))

    if cfg.plant_full_key:
        # full keys of the needle tokens = 3x the query of the group's first head
        for b in range(B):
            for r in range(R):
                kv = int(ret[r]) // G
                kn = f64_to_bf16_bits(3.0 * bf16_bits_to_f32(q[b, kv * G]).astype(np.float64))
                for j in needles[(b, r)]:
                    k_cache[b, kv, j * cfg.block:min(int(seq_lens[b]), (j + 1) * cfg.block)] = kn

    return DecodeInputs(cfg=cfg, seq_lens=seq_lens, ret_heads=ret, loc_heads=loc, top_p=top_p,
                        q=q, w_q=w_q, w_k=w_k, k_cache=k_cache, v_cache=v_cache, k_idx=k_idx,
                        needles=needles, peaked=peaked)


# ------------------------------------------------------------------ prefill inputs
@dataclasses.dataclass
class PrefillInputs:
    """The prompt of a prefill pass: every position's query, key and value rows."""
    cfg: DecodeConfig
    seq_lens: np.ndarray      # int32 [B]: prompt lengths N_b
    ret_heads: np.ndarray     # int32 [n_ret], ascending query-head ids
    loc_heads: np.ndarray     # int32 [n_loc]
    q: np.ndarray             # bf16 bits [B, Hq, T, 128]: row i = the query at position i
    k: np.ndarray             # bf16 bits [B, Hkv, T, 128]: the prompt's keys (no RoPE here, so also k_pre)
    v: np.ndarray             # bf16 bits [B, Hkv, T, 128]
    w_k: np.ndarray           # bf16 bits [n_ret, 16, 128]


def make_prefill_inputs(cfg: DecodeConfig, seed: Optional[int] = None, pad_value: int = 0,
                        workers: Optional[int] = None) -> PrefillInputs:
    """Seeded prompt for ``cfg``: T = max_ctx rows per head, the first N_b = ctx[b]
    of them drawn from N(0, 1) (queries, keys and values alike), the rest
    ``pad_value``.  Retrieval heads and W^K follow make_inputs' streams."""
    s = cfg.seed if seed is None else seed
    B, Hkv, Hq, R, Tm = cfg.B, cfg.Hkv, cfg.Hq, cfg.n_ret, cfg.max_ctx
    assert Hq % Hkv == 0 and 0 <= R <= Hq and len(cfg.ctx) == B and all(1 <= n for n in cfg.ctx)
    seq_lens = np.asarray(cfg.ctx, dtype=np.int32)
    if cfg.ret_heads is not None:
        ret = np.asarray(sorted(cfg.ret_heads), dtype=np.int32)
    else:
        ret = np.sort(_rng(s, _T_HEADS).choice(Hq, size=R, replace=False)).astype(np.int32)
    assert len(ret) == R
    loc = np.asarray([h for h in range(Hq) if h not in set(ret.tolist())], dtype=np.int32)
    wscale = np.float32(1.0 / np.sqrt(HEAD_DIM))
    w_k = np.empty((R, INDEX_DIM, HEAD_DIM), np.uint16)
    for r in range(R):
        w_k[r] = f32_to_bf16_bits(_rng(s, _T_WK, r).standard_normal((INDEX_DIM, HEAD_DIM), dtype=np.float32) * wscale)
    q = np.full((B, Hq, Tm, HEAD_DIM), pad_value, np.uint16)
    k = np.full((B, Hkv, Tm, HEAD_DIM), pad_value, np.uint16)
    v = np.full((B, Hkv, Tm, HEAD_DIM), pad_value, np.uint16)
    jobs = []
    for b in range(B):
        n = int(seq_lens[b])
        jobs += [(q[b, h], (s, _T_PQ, b, h), n) for h in range(Hq)]
        jobs += [(k[b, g], (s, _T_K, b, g), n) for g in range(Hkv)]
        jobs += [(v[b, g], (s, _T_V, b, g), n) for g in range(Hkv)]
    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(lambda a: _fill_normal(a[0], a[1], a[2], HEAD_DIM), jobs))
    return PrefillInputs(cfg=cfg, seq_lens=seq_lens, ret_heads=ret, loc_heads=loc, q=q, k=k, v=v, w_k=w_k)


def prefill_to_device(pin: PrefillInputs, device="cuda") -> Dict[str, "object"]:
    """Upload a prompt as torch tensors (bf16 tensors keep their bit patterns)."""
    import torch

    def bf(a: np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)

    def i32(a: np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return {"q": bf(pin.q), "k": bf(pin.k), "v": bf(pin.v), "w_k": bf(pin.w_k),
            "seq_lens": i32(pin.seq_lens), "ret_heads": i32(pin.ret_heads)}


def custom_config(name: str = "custom", **kw) -> DecodeConfig:
    """A workload with explicit shapes (for tests); unspecified fields take small defaults."""
    base = dict(seed=11, B=1, Hkv=1, Hq=4, n_ret=2, ctx=(1000,), block=64, top_p=None,
                window=64, sinks=4, split_tokens=256, kind="random")
    base.update(kw)
    if base["top_p"] is None:
        base["top_p"] = (0.9,) * base["n_ret"]
    base["ctx"] = tuple(int(v) for v in base["ctx"])
    base["top_p"] = tuple(float(v) for v in base["top_p"])
    return DecodeConfig(name=name, **base)


def to_device(inp: DecodeInputs, device="cuda") -> Dict[str, "object"]:
    """Upload the inputs as torch tensors (bf16 tensors keep their bit patterns)."""
    import torch

    def bf(a: np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)

    def i32(a: np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    q = bf(inp.q)
    return {
        "q": q, "q_pre": q, "w_q": bf(inp.w_q), "k_idx": bf(inp.k_idx),
        "k_cache": bf(inp.k_cache), "v_cache": bf(inp.v_cache),
        "seq_lens": i32(inp.seq_lens), "ret_heads": i32(inp.ret_heads), "loc_heads": i32(inp.loc_heads),
        "top_p": torch.from_numpy(np.ascontiguousarray(inp.top_p, dtype=np.float32)).to(device),
    }
