"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Block sets must pass the acceptance rule (bit-exact except within 1e-6 of the
threshold); outputs must be within max-abs 1e-2 and mean-rel 1e-3 of the oracle
(bf16 inputs, fp32 accumulation on the device)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Run, check_outputs, check_selection, say
from long_context_sparse_amd import DecodeStep, abi
from oracle import accept as A
from oracle import rtp_oracle as O

pytestmark = pytest.mark.gpu


def test_tiny_workload_all_heads():
    inp = W.make_inputs(W.get_config("tiny"))
    run = Run(inp)
    differ = check_selection(run)
    assert not differ, differ
    for r in range(4):   # both planted needle blocks, nothing else
        assert run.gpu_blocks(0, r).tolist() == inp.needles[(0, r)]
    check_outputs(run)


EDGE = [
    dict(name="ragged", B=3, Hkv=2, Hq=8, n_ret=3, ctx=(1000, 63, 4097), block=64, window=100, sinks=4,
         split_tokens=256, kind="peaked_diffuse"),
    dict(name="block128", B=3, Hkv=2, Hq=8, n_ret=3, ctx=(5000, 129, 128), block=128, window=300, sinks=2,
         split_tokens=512, kind="peaked_diffuse"),
    dict(name="p_one_dense", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(3001, 700), block=64, window=64, sinks=4,
         split_tokens=1024, kind="peaked_diffuse", top_p=(1.0, 1.0, 1.0, 1.0)),
    dict(name="all_retrieval", B=2, Hkv=2, Hq=8, n_ret=8, ctx=(2000, 1500), block=64, window=64, sinks=4,
         split_tokens=512, kind="peaked_diffuse"),
    dict(name="all_local", B=2, Hkv=2, Hq=8, n_ret=0, ctx=(2000, 1500), block=64, window=700, sinks=4,
         split_tokens=512, top_p=()),
    dict(name="window_covers_ctx", B=2, Hkv=1, Hq=4, n_ret=1, ctx=(3000, 5), block=64, window=10000, sinks=4,
         split_tokens=1024),
    dict(name="window1_nosink", B=2, Hkv=1, Hq=4, n_ret=1, ctx=(3000, 17), block=64, window=1, sinks=0,
         split_tokens=1024),
    dict(name="sinks_only", B=1, Hkv=1, Hq=4, n_ret=1, ctx=(3000,), block=64, window=0, sinks=7,
         split_tokens=1024),
    dict(name="single_token", B=2, Hkv=1, Hq=4, n_ret=2, ctx=(1, 2), block=64, window=8, sinks=4,
         split_tokens=64),
    dict(name="gqa1", B=1, Hkv=4, Hq=4, n_ret=2, ctx=(2500,), block=64, window=128, sinks=4, split_tokens=512,
         kind="peaked_diffuse"),
    dict(name="gqa2", B=1, Hkv=4, Hq=8, n_ret=3, ctx=(2500,), block=128, window=128, sinks=4, split_tokens=512,
         kind="peaked_diffuse"),
    dict(name="gqa8", B=2, Hkv=2, Hq=16, n_ret=9, ctx=(2500, 1900), block=64, window=200, sinks=4,
         split_tokens=512, kind="peaked_diffuse"),
    dict(name="low_p", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(4096, 3000), block=64, window=64, sinks=4,
         split_tokens=1024, top_p=(0.1, 0.3, 0.5, 0.7)),
    dict(name="high_p", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(4096, 3000), block=64, window=64, sinks=4,
         split_tokens=1024, kind="peaked_diffuse", top_p=(0.99, 0.999, 0.9999, 0.99999)),
    dict(name="needle_ties", B=1, Hkv=1, Hq=4, n_ret=2, ctx=(2048,), block=64, window=32, sinks=4,
         split_tokens=256, kind="needles3x", needles=(8, 8), top_p=(0.49, 0.3)),
    dict(name="many_splits", B=1, Hkv=2, Hq=8, n_ret=2, ctx=(20000,), block=64, window=5000, sinks=4,
         split_tokens=64, kind="peaked_diffuse"),
    # thousands of exactly equal block masses: resolved by count in ascending block order
    dict(name="flat_ties", B=2, Hkv=1, Hq=4, n_ret=3, ctx=(200000, 130000), block=64, window=64, sinks=4,
         split_tokens=4096, kind="flat", top_p=(0.3, 0.5, 0.77)),
    # near ties spread over a tiny mass range: several refinement levels
    dict(name="near_flat", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(300000, 77777), block=64, window=64, sinks=4,
         split_tokens=4096, kind="near_flat", top_p=(0.5, 0.9, 0.95, 0.99)),
    # the largest context a sequence may have at block 128 and one at block 64
    dict(name="max_blocks_128", B=1, Hkv=1, Hq=4, n_ret=2, ctx=(2097152,), block=128, window=256, sinks=4,
         split_tokens=65536, kind="peaked_diffuse"),
]


@pytest.mark.parametrize("spec", EDGE, ids=[e["name"] for e in EDGE])
def test_edge_workloads(spec):
    spec = dict(spec)
    name = spec.pop("name")
    cfg = W.custom_config(name=name, **spec)
    inp = W.make_inputs(cfg)
    run = Run(inp, tag=name)
    differ = check_selection(run)
    say(f"      {len(differ)} (b, r) sets differ inside the tie band")
    check_outputs(run)
    if name == "p_one_dense":
        for b in range(cfg.B):
            for r in range(cfg.n_ret):
                nblk = -(-int(inp.seq_lens[b]) // cfg.block)
                assert run.gpu_blocks(b, r).tolist() == list(range(nblk))
    if name == "flat_ties":
        # equal masses are admitted in ascending block order: the selection is a prefix
        for b in range(cfg.B):
            for r in range(cfg.n_ret):
                G = run.gpu_blocks(b, r)
                assert G.tolist() == list(range(len(G)))
    if name == "needle_ties":
        # 8 needles of bit-identical mass; ties are admitted in ascending block id
        for r, p in enumerate(cfg.top_p):
            k = int(np.ceil(p * 8))
            assert run.gpu_blocks(0, r).tolist() == sorted(inp.needles[(0, r)])[:k]


def test_split_partials_match_oracle():
    cfg = W.custom_config(name="partials", B=2, Hkv=2, Hq=8, n_ret=3, ctx=(3000, 2100), block=64, window=64,
                          sinks=4, split_tokens=512, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    run = Run(inp, tag="partials")
    o_part = run.step.o_part.cpu().numpy()
    lse_part = run.step.lse_part.cpu().numpy()
    n_split = o_part.shape[2]
    for b in range(cfg.B):
        n = int(inp.seq_lens[b])
        for r in range(cfg.n_ret):
            h = int(inp.ret_heads[r])
            kv = h // cfg.gqa
            toks = O.block_tokens(run.gpu_blocks(b, r), cfg.block, n)
            for c in range(n_split):
                tc = toks[(toks >= c * cfg.split_tokens) & (toks < (c + 1) * cfg.split_tokens)]
                o, lse = O.attend(inp.q[b, h], inp.k_cache[b, kv], inp.v_cache[b, kv], tc)
                if tc.size == 0:
                    assert lse_part[b, r, c] == -np.inf and not o_part[b, r, c].any()
                else:
                    assert abs(lse_part[b, r, c] - lse) < 1e-4 * max(1.0, abs(lse))
                    assert np.max(np.abs(o_part[b, r, c] - o)) < 1e-3


def test_split_size_does_not_change_result():
    cfg = W.custom_config(name="splits", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(6000, 4100), block=64, window=64,
                          sinks=4, split_tokens=6016, kind="peaked_diffuse", top_p=(1.0, 0.99, 0.95, 1.0))
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    one = Run(inp, tensors=t, split_tokens=6016, tag="one split")
    many = Run(inp, tensors=t, split_tokens=256, tag="24 splits")
    rows = [(b, int(h)) for b in range(cfg.B) for h in inp.ret_heads]
    a = np.stack([one.out_h[b, h] for b, h in rows])
    c = np.stack([many.out_h[b, h] for b, h in rows])
    assert np.max(np.abs(a - c)) < 1e-5


def test_nan_padding_is_never_read():
    cfg = W.custom_config(name="nanpad", B=3, Hkv=2, Hq=8, n_ret=3, ctx=(1000, 63, 4097), block=64,
                          window=100, sinks=4, split_tokens=256, kind="peaked_diffuse")
    inp = W.make_inputs(cfg, pad_value=int(W.BF16_NAN))
    run = Run(inp, tag="nan padding")
    assert np.all(np.isfinite(run.out_h))
    check_selection(run)
    check_outputs(run)


def test_unselected_blocks_are_never_read():
    cfg = W.custom_config(name="poison", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(5000, 3333), block=64, window=64,
                          sinks=4, split_tokens=1024, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    run = Run(inp, tensors=t, tag="poison: index pass")
    # poison every K/V row of every block no retrieval head of the group selected, then rerun
    # only the retrieval attention on the saved selection
    kc = t["k_cache"].clone()
    vc = t["v_cache"].clone()
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=kc.device)
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            keep = np.zeros(cfg.max_ctx, bool)
            for r, h in enumerate(inp.ret_heads):
                if int(h) // cfg.gqa == g:
                    for j in run.gpu_blocks(b, r):
                        keep[j * cfg.block:(j + 1) * cfg.block] = True
            rows = torch.from_numpy(np.nonzero(~keep)[0]).to(kc.device)
            kc[b, g, rows] = nan
            vc[b, g, rows] = nan
    t2 = dict(t, k_cache=kc, v_cache=vc)
    step = run.step
    step.out.zero_()
    say("[gpu] poison: sparse attention + reduce on poisoned caches")
    step.sparse_attn(t2)
    step.reduce(t2)
    torch.cuda.synchronize()
    out = step.out.cpu().numpy().astype(np.float64)
    for b in range(cfg.B):
        for r, h in enumerate(inp.ret_heads):
            assert np.all(np.isfinite(out[b, h]))
            ref = O.attend(inp.q[b, h], inp.k_cache[b, int(h) // cfg.gqa], inp.v_cache[b, int(h) // cfg.gqa],
                           O.block_tokens(run.gpu_blocks(b, r), cfg.block, int(inp.seq_lens[b])))[0]
            assert np.max(np.abs(out[b, h] - ref)) < 1e-2


def test_repeat_calls_are_deterministic():
    cfg = W.custom_config(name="determinism", B=2, Hkv=2, Hq=8, n_ret=4, ctx=(9000, 7777), block=64,
                          window=500, sinks=4, split_tokens=1024, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    run = Run(inp, tag="determinism")
    ref_out = run.out.clone()
    ref_sel = run.step.sel_idx.clone()
    ref_cnt = run.step.sel_cnt.clone()
    say("[gpu] determinism: 30 repeated steps")
    for _ in range(30):
        run.step(run.t)
    torch.cuda.synchronize()
    assert torch.equal(run.step.sel_cnt, ref_cnt)
    for b in range(cfg.B):
        for r in range(cfg.n_ret):
            k = int(ref_cnt[b, r])
            assert torch.equal(run.step.sel_idx[b, r, :k], ref_sel[b, r, :k])
    assert torch.equal(run.out, ref_out)


def test_workspace_reuse_across_inputs():
    """One DecodeStep (one pair of workspaces) over two different inputs, twice each."""
    cfg = W.custom_config(name="reuse", B=2, Hkv=2, Hq=8, n_ret=3, ctx=(4000, 2500), block=64, window=128,
                          sinks=4, split_tokens=512, kind="peaked_diffuse")
    a = W.make_inputs(cfg)
    b_ = W.make_inputs(cfg, seed=cfg.seed + 100)
    ra = Run(a, tag="reuse A")
    ta, tb = ra.t, W.to_device(b_)
    outs = []
    say("[gpu] reuse: alternate inputs on one step object")
    for t in (tb, ta, tb):
        outs.append(ra.step(t).clone())
    torch.cuda.synchronize()
    assert np.array_equal(outs[1].cpu().numpy().astype(np.float64), ra.out_h)
    rb = Run(b_, tensors=tb, tag="reuse B fresh")
    assert np.array_equal(outs[0].cpu().numpy().astype(np.float64), rb.out_h)
    assert np.array_equal(outs[2].cpu().numpy().astype(np.float64), rb.out_h)


def test_block_masks_match_lists_and_give_the_same_partials():
    """The index call's block masks hold exactly the listed blocks, and the split attention
    reading its union from the masks writes bit-identical partials to the list search."""
    cfg = W.custom_config(name="masks", B=3, Hkv=2, Hq=8, n_ret=6, ctx=(9000, 4097, 70), block=64, window=64,
                          sinks=4, split_tokens=512, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    m = Run(inp, tensors=t, tag="masks")
    ls = Run(inp, tensors=t, tag="lists", use_mask=False)
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
    assert torch.equal(m.step.lse_part, ls.step.lse_part)
    assert np.array_equal(m.out_h, ls.out_h)
    # masks alone (no lists, no counts): the KV groups go in their natural order and every
    # split's partials are the same bits
    o2 = torch.full_like(m.step.o_part, float("nan"))
    l2 = torch.full_like(m.step.lse_part, float("nan"))
    s = m.step.s
    abi.rtp_sparse_attn_split(t["q"], t["k_cache"], t["v_cache"], t["seq_lens"], t["ret_heads"], None, None,
                              s.B, s.Hq, s.Hkv, s.n_ret, s.max_ctx, s.block, s.split_tokens, o2, l2,
                              sel_mask=m.step.sel_mask)
    torch.cuda.synchronize()
    assert torch.equal(o2, m.step.o_part)
    assert torch.equal(l2, m.step.lse_part)


@pytest.mark.parametrize("n_ret,window,overlap", [(3, 8192, True), (3, 8192, False), (3, 600, True),
                                                  (0, 8192, True), (32, 600, True)])
def test_step_matches_the_four_calls(n_ret, window, overlap):
    """rtp_decode_step (index, one attention launch for both head kinds, one merge) against
    the four separate calls rtp_index_topp, rtp_sparse_attn_split, rtp_split_reduce and
    rtp_local_window_attn: the same block sets and the same output bits, with both head
    kinds (the local heads on the second stream: window 8192 over 8 KV heads and 2
    sequences, 67 MB of K/V; or in the attention launch: window 600, or no second stream
    given), with no retrieval heads, and with no local heads; both against the oracle."""
    cfg = W.custom_config(name=f"calls{n_ret}", B=2, Hkv=8, Hq=32, n_ret=n_ret, ctx=(20000, 9001), block=64,
                          window=window, sinks=4, split_tokens=1024, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    step = Run(inp, tensors=t, tag=f"step n_ret={n_ret} window={window} overlap={overlap}", overlap=overlap)
    calls = DecodeStep(step.step.s, overlap=False)
    out = torch.full_like(calls.out, float("nan"))
    calls.out = out
    if cfg.n_ret:
        calls.index_topp(t)
        calls.sparse_attn(t)
        calls.reduce(t)
    if cfg.n_loc:
        calls.local(t)
    torch.cuda.synchronize()
    sep = out.cpu().numpy().astype(np.float64)
    ret = [int(h) for h in inp.ret_heads]
    loc = [int(h) for h in inp.loc_heads]
    assert np.array_equal(sep[:, ret], step.out_h[:, ret])
    assert np.array_equal(sep[:, loc], step.out_h[:, loc])
    if cfg.n_ret:
        assert torch.equal(calls.sel_cnt.cpu(), torch.from_numpy(step.sel_cnt))
        check_selection(step)
    check_outputs(step)


def test_two_stream_step_tracks_changing_queries():
    """The step with the local heads on the second stream (ordered by the fork and join
    events) against the one-stream step, over 8 back-to-back steps whose queries change
    on the device before each one: outputs bit-identical and the same block sets at every
    step.  A join that let the merge read the previous step's local partials, or a fork
    that let the local heads read the previous queries, would show as a difference,
    since consecutive steps no longer share their inputs."""
    cfg = W.custom_config(name="fork_loop", B=2, Hkv=8, Hq=32, n_ret=3, ctx=(20000, 9001), block=64,
                          window=8192, sinks=4, split_tokens=1024, kind="peaked_diffuse")
    inp = W.make_inputs(cfg)
    t = W.to_device(inp)
    two = Run(inp, tensors=t, tag="fork_loop two streams", overlap=True)
    assert two.step.overlap and two.step.side is not None
    one = DecodeStep(two.step.s, overlap=False)
    gen = torch.Generator(device=t["q"].device).manual_seed(11)
    for i in range(8):
        # new queries for every head (the index and the attention read the same rows)
        qn = torch.randn(t["q"].shape, device=t["q"].device, generator=gen).to(torch.bfloat16)
        t["q"].copy_(qn)
        a = two.step(t).clone()
        b = one(t).clone()
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"step {i}: outputs differ between the two-stream and one-stream steps"
        assert torch.equal(two.step.sel_cnt, one.sel_cnt), f"step {i}: block counts differ"
        assert torch.equal(two.step.sel_idx, one.sel_idx), f"step {i}: block lists differ"
    say("      8 steps with changing queries: two-stream and one-stream steps bit-identical")
