"""GPU parity on the five named decode workloads at their full sizes, in the launch
configuration the benchmark times.  Every (sequence, retrieval head) selection is
checked against the oracle's masses; outputs are compared on every query head of every
sequence, retrieval and local (the oracle computes each row on its own)."""
import numpy as np
import pytest

import workloads as W
from gpu_util import Run, check_outputs, check_selection, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "ctx32k", "ctx128k", "ctx1m", "mixed"])
def test_named_workload(name):
    cfg = W.get_config(name)
    say(f"[gen] {name}")
    inp = W.make_inputs(cfg)
    run = Run(inp, tag=name)
    differ = check_selection(run)
    sel = [(b, r, int(run.sel_cnt[b, r])) for b in range(cfg.B) for r in range(cfg.n_ret)]
    frac = np.mean([c / -(-int(inp.seq_lens[b]) // cfg.block) for b, r, c in sel])
    say(f"      {len(differ)} sets differ inside the tie band; mean selected fraction {frac:.3f}")
    check_outputs(run)  # every (sequence, query head)
    if cfg.kind in ("depth_needles", "needles3x"):
        for (b, r), blocks in inp.needles.items():
            assert run.gpu_blocks(b, r).tolist() == sorted(blocks), (b, r)
