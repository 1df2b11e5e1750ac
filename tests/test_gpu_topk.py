"""GPU parity of the static top-k selection rule (rtp_index_topk, the review's fixed-
budget variant with k = 4096): block sets against the oracle's select_top_k (exact
size, bit-exact except ties within 1e-6 of the threshold mass), outputs against the
oracle's attention over the device's set, at the bench's full sizes and on edge cases."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Run, check_outputs, check_selection_topk, say

pytestmark = pytest.mark.gpu


def _items(inp):
    return [(b, int(h)) for b in range(inp.cfg.B) for h in inp.ret_heads]


@pytest.mark.parametrize("name", ["ctx32k", "ctx128k", "ctx1m"])
def test_topk_named_workload(name):
    cfg = W.get_config(name)
    say(f"[gen] {name}")
    inp = W.make_inputs(cfg)
    run = Run(inp, tag=f"{name} top-k", k_tokens=4096)
    differ = check_selection_topk(run)
    kb = -(-4096 // cfg.block)
    for b in range(cfg.B):
        nblk = -(-int(inp.seq_lens[b]) // cfg.block)
        assert np.all(run.sel_cnt[b, :cfg.n_ret] == min(kb, nblk))
    say(f"      {len(differ)} sets differ inside the tie band; {kb} blocks a head")
    check_outputs(run, _items(inp))


TOPK_EDGE = [
    # budget beyond the context (every block), one token (one block), ragged lengths
    dict(name="budget_covers", k_tokens=1 << 20, B=2, Hkv=2, Hq=8, n_ret=3, ctx=(3000, 65), block=64,
         split_tokens=512, kind="peaked_diffuse"),
    dict(name="one_block", k_tokens=1, B=2, Hkv=2, Hq=8, n_ret=3, ctx=(9000, 1), block=64, split_tokens=1024,
         kind="peaked_diffuse"),
    dict(name="block128", k_tokens=1000, B=3, Hkv=2, Hq=8, n_ret=3, ctx=(20000, 129, 1000), block=128,
         split_tokens=512, kind="peaked_diffuse"),
    # thousands of bit-identical masses: ties go to the lowest block ids
    dict(name="flat_ties", k_tokens=4096, B=1, Hkv=1, Hq=4, n_ret=2, ctx=(200000,), block=64,
         split_tokens=4096, kind="flat"),
    # near ties over a tiny mass range: several refinement levels with unit weights
    dict(name="near_flat", k_tokens=7000, B=2, Hkv=2, Hq=8, n_ret=4, ctx=(300000, 77777), block=64,
         split_tokens=4096, kind="near_flat"),
    dict(name="max_blocks", k_tokens=65536, B=1, Hkv=1, Hq=4, n_ret=2, ctx=(2097152,), block=128,
         split_tokens=65536, kind="peaked_diffuse"),
]


@pytest.mark.parametrize("spec", TOPK_EDGE, ids=[e["name"] for e in TOPK_EDGE])
def test_topk_edges(spec):
    spec = dict(spec)
    name, k_tokens = spec.pop("name"), spec.pop("k_tokens")
    cfg = W.custom_config(name=name, window=64, sinks=4, **spec)
    inp = W.make_inputs(cfg)
    run = Run(inp, tag=name, k_tokens=k_tokens)
    differ = check_selection_topk(run)
    say(f"      {len(differ)} (b, r) sets differ inside the tie band")
    check_outputs(run, _items(inp))
    kb = -(-k_tokens // cfg.block)
    for b in range(cfg.B):
        nblk = -(-int(inp.seq_lens[b]) // cfg.block)
        for r in range(cfg.n_ret):
            G = run.gpu_blocks(b, r)
            assert G.size == min(kb, nblk)
            if name == "budget_covers":
                assert G.tolist() == list(range(nblk))
            if name == "flat_ties":
                assert G.tolist() == list(range(min(kb, nblk)))


def test_topk_masks_match_lists():
    """The block masks rtp_index_topk writes hold exactly its lists, and the split
    attention gives the same bits from either."""
    cfg = W.custom_config(name="topk_masks", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(30000, 7001), block=64, window=64,
                          sinks=4, split_tokens=1024, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    m = Run(inp, tensors=t, tag="top-k masks", k_tokens=2048)
    ls = Run(inp, tensors=t, tag="top-k lists", use_mask=False, k_tokens=2048)
    mask = m.step.sel_mask.cpu().numpy()
    for b in range(cfg.B):
        nblk = -(-int(inp.seq_lens[b]) // cfg.block)
        for r in range(cfg.n_ret):
            G = m.gpu_blocks(b, r)
            assert np.array_equal(G, ls.gpu_blocks(b, r))
            want = np.zeros(nblk, np.uint8)
            want[G] = 1
            assert np.array_equal(mask[b, r, :nblk], want), (b, r)
    assert torch.equal(m.step.o_part, ls.step.o_part)
    assert np.array_equal(m.out_h, ls.out_h)
