"""Host logic of bench.py (CPU): the algorithmic byte and flop counts its rooflines
divide by, the traffic records it reads, and the one-GPU guard."""
import os
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import rtp_oracle as O  # noqa: E402


@pytest.mark.parametrize("N,W,S", [(1, 8, 4), (100, 7, 2), (300, 64, 4), (50, 100, 4), (1000, 64, 0), (33, 0, 5)])
def test_prefill_flops_counts_attended_pairs(N, W, S):
    ret_pairs = sum(len(O.prefill_tokens(i, True, W, S)) for i in range(N))
    loc_pairs = sum(len(O.prefill_tokens(i, False, W, S)) for i in range(N))
    assert bench.prefill_flops(N, 1, 0, W, S) == 512 * ret_pairs
    assert bench.prefill_flops(N, 0, 1, W, S) == 512 * loc_pairs
    assert bench.prefill_flops(N, 3, 5, W, S) == 512 * (3 * ret_pairs + 5 * loc_pairs)


def test_algorithmic_bytes_hand_worked():
    # one sequence of 300 tokens, one KV head with query heads 0 (retrieval) and 1 (local);
    # blocks 0 and 4 selected (tokens 0-63 and 256-299: 108 tokens), window 64 + 4 sinks
    # (tokens 0-3 and 236-299: 68 tokens); their union is 0-63 and 236-299 (128 tokens)
    cfg = types.SimpleNamespace(B=1, Hq=2, Hkv=1, block=64, window=64, sinks=4)
    inp = types.SimpleNamespace(ret_heads=np.array([0]), loc_heads=np.array([1]), seq_lens=np.array([300]))
    sel_idx = np.array([[[0, 4, 0, 0, 0]]])
    sel_cnt = np.array([[2]])
    a = bench.algorithmic_bytes(cfg, inp, sel_idx, sel_cnt)
    assert a["index_topp"] == 4096 + 32 * 300 + 256 + 4 * 2 + 4
    assert a["decode_attn"] == 512 * 128 + 256 * 2          # the union once, both query rows
    assert a["decode_merge"] == 512 * 2                      # both fp32 output rows
    assert a["kv_rows_selected_union"] == 108 and a["kv_rows_window"] == 68
    assert a["step"] == a["index_topp"] + a["decode_attn"] + a["decode_merge"]


def test_traffic_record_follows_kernel_sources(monkeypatch):
    # the committed record is read while its sources are unchanged, and dropped after
    rec = bench.read_traffic("ctx128k", "decode_attn")
    if rec is None:
        pytest.skip("no current traffic record for the step's attention launch at 128K")
    assert rec > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel: "0" * 16)
    assert bench.read_traffic("ctx128k", "decode_attn") is None


def test_kernel_source_hash_covers_included_headers(tmp_path, monkeypatch):
    csrc = tmp_path / "long_context_sparse_amd" / "csrc"
    inc = tmp_path / "include"
    csrc.mkdir(parents=True)
    inc.mkdir()
    (csrc / "k.hip").write_text('#include "a.hpp"\n')
    (csrc / "a.hpp").write_text('#include "rtp.h"\nint x;\n')
    (inc / "rtp.h").write_text("int y;\n")
    (csrc / "other.hip").write_text("int z;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCE, "k_kernel", "k.hip")
    h0 = bench.kernel_source_hash("k_kernel")
    (csrc / "other.hip").write_text("int z2;\n")       # not included: same hash
    assert bench.kernel_source_hash("k_kernel") == h0
    (inc / "rtp.h").write_text("int y2;\n")            # included through a.hpp: new hash
    assert bench.kernel_source_hash("k_kernel") != h0


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err
