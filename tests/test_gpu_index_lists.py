"""GPU parity of the index selection where the chunks' heavy-block lists decide it.

Under the top-p rule, with more than 2048 blocks in a sequence and at most 128 chunks a
head, every chunk publishes the blocks that hold at least 1/8 of its own mass.  The
selecting workgroup first ranks the listed blocks whose mass exceeds U, the largest bound
fl(fl(Z_c / 8) f_c) on an unlisted block.  When they reach p, that prefix is the selection.
Otherwise the full pass decides.  Both outcomes must give the oracle's block sets (the
greedy top-p prefix of the Review, Adaptive sparse attention; exact up to the tie band).
The cases mix heads that the lists decide (planted needles, peaked heads, bit-identical
needle ties cut by p) with heads they cannot decide (diffuse heads, short sequences
below the size limit), in both index-kernel builds (grids of at most one workgroup per
compute unit and larger ones).
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import Run, check_outputs, check_selection, say
from oracle import rtp_oracle as O

pytestmark = pytest.mark.gpu

CUS = 256  # compute units of the MI355X: the index grid's chunking target


def chunk_blocks(B: int, n_ret: int, max_ctx: int, block: int, T: int = 1024, target: int = CUS) -> int:
    """The index kernel's chunk size in blocks for this batch: at least `target`
    workgroups where the blocks allow, 8..256 blocks a chunk, at most 2 T chunks a head."""
    nblk_max = -(-max_ctx // block)
    total = B * n_ret * nblk_max
    cb = 256
    while cb > 8 and total // cb < target:
        cb >>= 1
    while -(-nblk_max // cb) > 2 * T and cb < 256:
        cb <<= 1
    return cb


def lists_decide(m: np.ndarray, p: float, cb: int) -> bool:
    """Host model (fp64 masses) of whether the listed blocks decide a head's selection."""
    nblk = len(m)
    nch = -(-nblk // cb)
    if nblk <= 2048 or nch > 128 or p >= 1.0:
        return False
    U, listed = 0.0, []
    for c in range(nch):
        seg = m[c * cb:(c + 1) * cb]
        zc = float(seg.sum())
        U = max(U, zc / 8)
        listed += [float(x) for x in seg if x >= zc / 8]
    above = sorted((x for x in listed if x > U), reverse=True)
    return bool(above) and float(np.sum(above)) >= p


CASES = [
    # planted needles (1..8 a head), two sequences, grid over one workgroup per unit
    dict(name="lists_needles", B=2, Hkv=2, Hq=8, n_ret=3, ctx=(300000, 200000), block=64, window=256, sinks=4,
         split_tokens=8192, kind="needles3x", needles=(1, 8), top_p=(0.9, 0.95, 0.99)),
    # needles at depths 0.1 / 0.5 / 0.9, block 128, one workgroup per unit
    dict(name="lists_depth", B=1, Hkv=2, Hq=8, n_ret=2, ctx=(524288,), block=128, window=1024, sinks=4,
         split_tokens=65536, kind="depth_needles", top_p=(0.95, 0.5)),
    # peaked and diffuse heads, one sequence below the size limit
    dict(name="lists_mixed", B=3, Hkv=2, Hq=8, n_ret=2, ctx=(262144, 150000, 4000), block=64, window=512, sinks=4,
         split_tokens=8192, kind="peaked_diffuse", top_p=(0.5, 0.99)),
    # eight needles of bit-identical mass, p cutting through them: ties by ascending id
    dict(name="lists_ties", B=1, Hkv=1, Hq=4, n_ret=4, ctx=(134400,), block=64, window=64, sinks=4,
         split_tokens=4096, kind="needles3x", needles=(8, 8), top_p=(0.49, 0.3, 0.9, 0.2)),
]


@pytest.mark.parametrize("spec", CASES, ids=[c["name"] for c in CASES])
def test_index_lists_selection(spec):
    spec = dict(spec)
    name = spec.pop("name")
    cfg = W.custom_config(name=name, **spec)
    inp = W.make_inputs(cfg)
    cb = chunk_blocks(cfg.B, cfg.n_ret, cfg.max_ctx, cfg.block)
    decidable = [(b, r) for b in range(cfg.B) for r in range(cfg.n_ret)
                 if lists_decide(O.retrieval_masses(inp, b, r), float(inp.top_p[b, r]), cb)]
    say(f"      chunk {cb} blocks; heads the lists decide (host model): {len(decidable)} of {cfg.B * cfg.n_ret}")
    assert decidable, "the case should exercise the lists"
    run = Run(inp, tag=name)
    differ = check_selection(run)
    say(f"      {len(differ)} (b, r) sets differ inside the tie band")
    check_outputs(run)
    if name == "lists_ties":
        for r, p in enumerate(cfg.top_p):
            k = int(np.ceil(p * 8))
            assert run.gpu_blocks(0, r).tolist() == sorted(inp.needles[(0, r)])[:k]
