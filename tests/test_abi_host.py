"""Host side of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before touching a device."""
import ctypes

import pytest

from long_context_sparse_amd import abi

FAKE = 4096  # a non-null, 256-aligned stand-in pointer; never dereferenced on these paths


def test_exports_every_declared_symbol():
    L = abi.lib()
    names = abi.declared_functions()
    assert {"rtp_index_topp", "rtp_sparse_attn_split", "rtp_split_reduce", "rtp_local_window_attn"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert abi.status_string(0) == "RTP_OK"
    assert "EINVAL" in abi.status_string(1)
    assert "EUNSUPPORTED" in abi.status_string(2)
    assert "ELAUNCH" in abi.status_string(3)
    assert "gfx950" in abi.version()


def test_workspace_sizes():
    s = abi.rtp_index_topp_workspace_size(4, 8, 131072, 64)
    assert s >= 4 * 8 * 2048 * 8          # one fp64 per block at least
    assert abi.rtp_index_topp_workspace_size(4, 8, 131072, 32) == 0
    assert abi.rtp_index_topp_workspace_size(0, 8, 131072, 64) == 0
    assert abi.rtp_local_window_workspace_size(4, 32, 8, 24, 131072, 8192, 4) > 0
    assert abi.rtp_local_window_workspace_size(4, 32, 8, 24, 131072, 0, 0) == 0


def _topp(**kw):
    a = dict(q_pre=FAKE, w_q=FAKE, k_idx=FAKE, seq_lens=FAKE, ret_heads=FAKE, top_p=FAKE, B=1, Hq=4,
             n_ret=2, max_ctx=1024, block=64, sel_idx=FAKE, sel_cnt=FAKE, sel_mask=None, ws=FAKE, ws_bytes=0,
             stream=None)
    a.update(kw)
    if a["ws_bytes"] == 0 and "ws_bytes" not in kw:
        a["ws_bytes"] = abi.rtp_index_topp_workspace_size(a["B"], a["n_ret"], a["max_ctx"], a["block"]) - 1
    return abi.lib().rtp_index_topp(a["q_pre"], a["w_q"], a["k_idx"], a["seq_lens"], a["ret_heads"], a["top_p"],
                                    a["B"], a["Hq"], a["n_ret"], a["max_ctx"], a["block"], a["sel_idx"],
                                    a["sel_cnt"], a["sel_mask"], a["ws"], a["ws_bytes"], a["stream"])


def test_index_topp_rejects():
    assert _topp() == abi.RTP_EINVAL                    # workspace one byte short
    assert _topp(block=32) == abi.RTP_EUNSUPPORTED
    assert _topp(block=256) == abi.RTP_EUNSUPPORTED
    assert _topp(B=0) == abi.RTP_EINVAL
    assert _topp(n_ret=5) == abi.RTP_EINVAL             # more retrieval heads than heads
    assert _topp(max_ctx=0) == abi.RTP_EINVAL
    assert _topp(q_pre=None, ws_bytes=1 << 30) == abi.RTP_EINVAL
    assert _topp(k_idx=FAKE + 2, ws_bytes=1 << 30) == abi.RTP_EINVAL   # misaligned
    assert _topp(ws=FAKE + 16, ws_bytes=1 << 30) == abi.RTP_EINVAL    # workspace not 256-aligned
    assert _topp(n_ret=0) == abi.RTP_OK                 # no-op


def _topk(k_tokens=4096, **kw):
    a = dict(q_pre=FAKE, w_q=FAKE, k_idx=FAKE, seq_lens=FAKE, ret_heads=FAKE, B=1, Hq=4,
             n_ret=2, max_ctx=1024, block=64, sel_idx=FAKE, sel_cnt=FAKE, sel_mask=None, ws=FAKE, ws_bytes=0)
    a.update(kw)
    if "ws_bytes" not in kw:
        a["ws_bytes"] = abi.rtp_index_topp_workspace_size(a["B"], a["n_ret"], a["max_ctx"], a["block"]) - 1
    return abi.lib().rtp_index_topk(a["q_pre"], a["w_q"], a["k_idx"], a["seq_lens"], a["ret_heads"], k_tokens,
                                    a["B"], a["Hq"], a["n_ret"], a["max_ctx"], a["block"], a["sel_idx"],
                                    a["sel_cnt"], a["sel_mask"], a["ws"], a["ws_bytes"], None)


def test_index_topk_rejects():
    assert _topk() == abi.RTP_EINVAL                    # workspace one byte short
    assert _topk(k_tokens=0, ws_bytes=1 << 30) == abi.RTP_EINVAL
    assert _topk(k_tokens=-5, ws_bytes=1 << 30) == abi.RTP_EINVAL
    assert _topk(block=32, ws_bytes=1 << 30) == abi.RTP_EUNSUPPORTED
    assert _topk(B=0, ws_bytes=1 << 30) == abi.RTP_EINVAL
    assert _topk(q_pre=None, ws_bytes=1 << 30) == abi.RTP_EINVAL
    assert _topk(k_idx=FAKE + 2, ws_bytes=1 << 30) == abi.RTP_EINVAL
    assert _topk(n_ret=0) == abi.RTP_OK                 # no-op


def _sparse(**kw):
    a = dict(B=1, Hq=8, Hkv=2, n_ret=2, max_ctx=4096, block=64, split=1024, sel_idx=FAKE, sel_cnt=FAKE,
             sel_mask=None, kv_slot=None, n_full=0)
    a.update(kw)
    ptr = kw.get("ptr", FAKE)
    return abi.lib().rtp_sparse_attn_split(ptr, FAKE, FAKE, FAKE, FAKE, a["sel_idx"], a["sel_cnt"], a["sel_mask"],
                                           a["B"], a["Hq"], a["Hkv"], a["n_ret"], a["max_ctx"], a["block"],
                                           a["split"], FAKE, FAKE, a["kv_slot"], a["n_full"], None)


def test_sparse_attn_rejects():
    assert _sparse(split=100) == abi.RTP_EINVAL           # not a multiple of the block
    assert _sparse(split=0) == abi.RTP_EINVAL
    assert _sparse(block=96) == abi.RTP_EUNSUPPORTED
    assert _sparse(Hq=8, Hkv=3) == abi.RTP_EINVAL         # heads not divisible
    assert _sparse(Hq=48, Hkv=2) == abi.RTP_EUNSUPPORTED  # 24 query heads per KV head
    assert _sparse(split=64 * 4096) == abi.RTP_EUNSUPPORTED
    assert _sparse(ptr=None) == abi.RTP_EINVAL
    assert _sparse(sel_idx=None) == abi.RTP_EINVAL          # no lists and no masks
    assert _sparse(sel_cnt=None) == abi.RTP_EINVAL
    assert _sparse(kv_slot=FAKE, n_full=0) == abi.RTP_EINVAL   # placement without full caches
    assert _sparse(kv_slot=FAKE, n_full=3) == abi.RTP_EINVAL   # more full slots than groups
    assert _sparse(n_ret=0) == abi.RTP_OK


def test_reduce_and_local_reject():
    L = abi.lib()
    assert L.rtp_split_reduce(FAKE, FAKE, FAKE, 1, 4, 5, 2, FAKE, None) == abi.RTP_EINVAL
    assert L.rtp_split_reduce(FAKE, FAKE, FAKE, 1, 4, 2, 0, FAKE, None) == abi.RTP_EINVAL
    assert L.rtp_split_reduce(None, FAKE, FAKE, 1, 4, 2, 2, FAKE, None) == abi.RTP_EINVAL
    assert L.rtp_split_reduce(FAKE, FAKE, FAKE, 1, 4, 0, 2, FAKE, None) == abi.RTP_OK
    ws = abi.rtp_local_window_workspace_size(1, 8, 2, 6, 4096, 1024, 4)
    nop = [None, 0, None, None, 0, None]            # no placement table; default stream

    def loc(window=1024, sinks=4, n_loc=6, ws_bytes=1 << 30, kc=FAKE, tail=nop):
        return L.rtp_local_window_attn(FAKE, kc, kc, FAKE, FAKE, 1, 8, 2, n_loc, 4096, window, sinks, FAKE,
                                       FAKE, ws_bytes, *tail)
    assert loc(ws_bytes=ws - 1) == abi.RTP_EINVAL
    assert loc(window=0, sinks=0) == abi.RTP_EINVAL
    assert loc(window=-1) == abi.RTP_EINVAL
    assert loc(kc=None) == abi.RTP_EINVAL                         # no caches at all
    assert loc(tail=[FAKE, 0, None, None, 0, None]) == abi.RTP_EINVAL      # placement with no groups
    assert loc(tail=[FAKE, 1, None, None, 1, None]) == abi.RTP_EINVAL      # rings missing
    assert loc(tail=[FAKE, 1, FAKE + 4, FAKE, 1, None]) == abi.RTP_EINVAL  # ring misaligned
    assert loc(kc=None, tail=[FAKE, 1, FAKE, FAKE, 1, None]) == abi.RTP_EINVAL  # full slots, no caches
    assert loc(tail=[FAKE, 3, None, None, 0, None]) == abi.RTP_EINVAL      # more full slots than groups
    assert loc(n_loc=0, window=16, ws_bytes=0) == abi.RTP_OK


def test_cache_append_rejects():
    L = abi.lib()

    def call(B=2, Hq=8, Hkv=2, n_ret=2, max_ctx=256, k_new=FAKE, k_pre=FAKE, k_idx=FAKE,
             place=(None, 0, None, None, 0, 0, 0)):
        return L.rtp_cache_append(k_new, FAKE, k_pre, FAKE, FAKE, FAKE, B, Hq, Hkv, n_ret, max_ctx,
                                  FAKE, FAKE, k_idx, *place, None)
    assert call(B=0) == abi.RTP_EINVAL
    assert call(Hkv=3) == abi.RTP_EINVAL                 # heads not divisible
    assert call(n_ret=9) == abi.RTP_EINVAL               # more retrieval heads than heads
    assert call(max_ctx=0) == abi.RTP_EINVAL
    assert call(k_new=None) == abi.RTP_EINVAL
    assert call(k_pre=None) == abi.RTP_EINVAL            # needed for the index keys
    assert call(k_new=FAKE + 8) == abi.RTP_EINVAL        # misaligned
    assert call(k_idx=FAKE + 1) == abi.RTP_EINVAL
    assert call(place=(FAKE, 1, FAKE, FAKE, 1, 0, 0)) == abi.RTP_EINVAL      # ring of no rows
    assert call(place=(FAKE, 1, None, FAKE, 1, 4, 16)) == abi.RTP_EINVAL     # ring missing
    assert call(place=(FAKE, 2, FAKE, FAKE, 1, 4, 16)) == abi.RTP_EINVAL     # 3 slots for 2 groups
    assert call(place=(FAKE, 1, FAKE, FAKE, 1, -1, 16)) == abi.RTP_EINVAL


def test_decode_step_rejects():
    L = abi.lib()
    args = [FAKE] * 10 + [0] + [1, 8, 2, 2, 6, 4096, 64, 1024, 1024, 4] + [FAKE] * 6 + \
        [FAKE, 1 << 30, FAKE, 1 << 30] + [None, 0, None, None, 0] + [None] * 4
    bad = list(args)
    bad[11] = 0                                        # B = 0
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL
    bad = list(args)
    bad[14], bad[15] = 5, 6                            # more heads than query heads
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL
    bad = list(args)
    bad[17] = 96                                       # block size outside {64, 128}
    assert L.rtp_decode_step(*bad) == abi.RTP_EUNSUPPORTED
    bad = list(args)
    bad[10] = -1                                       # negative top-k budget
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL
    bad = list(args)
    bad[9] = None                                      # top-p rule without top_p
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL
    bad = list(args)
    bad[31:36] = [FAKE, 0, FAKE, FAKE, 2]              # retrieval heads but no full caches
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL
    bad = list(args)
    bad[31:36] = [FAKE, 1, None, None, 1]              # ring groups but no rings
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL
    bad = list(args)
    bad[31:36] = [FAKE, 2, FAKE, FAKE, 1]              # three slots for two groups
    assert L.rtp_decode_step(*bad) == abi.RTP_EINVAL


def test_prefill_rejects():
    L = abi.lib()

    def attn(B=1, Hq=8, Hkv=2, n_ret=2, max_ctx=4096, window=1024, sinks=4, q=FAKE, rh=FAKE):
        return L.rtp_prefill_attn(q, FAKE, FAKE, FAKE, rh, B, Hq, Hkv, n_ret, max_ctx, window, sinks, FAKE, None)
    assert attn(B=0) == abi.RTP_EINVAL
    assert attn(Hkv=3) == abi.RTP_EINVAL
    assert attn(n_ret=9) == abi.RTP_EINVAL
    assert attn(window=0, sinks=0) == abi.RTP_EINVAL       # local heads with an empty rule
    assert attn(window=-1) == abi.RTP_EINVAL
    assert attn(q=None) == abi.RTP_EINVAL
    assert attn(q=FAKE + 8) == abi.RTP_EINVAL               # misaligned
    assert attn(rh=None) == abi.RTP_EINVAL                  # retrieval heads without their list
    assert attn(max_ctx=1 << 30) == abi.RTP_EUNSUPPORTED     # more query tiles than a grid holds

    def keys(B=1, Hq=8, Hkv=2, n_ret=2, max_ctx=4096, k_pre=FAKE, k_idx=FAKE):
        return L.rtp_prefill_index_keys(k_pre, FAKE, FAKE, FAKE, B, Hq, Hkv, n_ret, max_ctx, k_idx, None)
    assert keys(B=0) == abi.RTP_EINVAL
    assert keys(Hkv=3) == abi.RTP_EINVAL
    assert keys(k_pre=None) == abi.RTP_EINVAL
    assert keys(k_pre=FAKE + 4) == abi.RTP_EINVAL
    assert keys(k_idx=FAKE + 1) == abi.RTP_EINVAL
    assert keys(n_ret=0) == abi.RTP_OK                      # no-op


def test_ring_fill_rejects():
    L = abi.lib()

    def fill(B=1, Hkv=2, max_ctx=4096, n_ring=1, sinks=4, window=16, k=FAKE, kr=FAKE):
        return L.rtp_ring_fill(k, FAKE, FAKE, FAKE, B, Hkv, max_ctx, kr, FAKE, n_ring, sinks, window, None)
    assert fill(B=0) == abi.RTP_EINVAL
    assert fill(n_ring=3) == abi.RTP_EINVAL             # more rings than groups
    assert fill(sinks=0, window=0) == abi.RTP_EINVAL    # a ring of no rows
    assert fill(window=-1) == abi.RTP_EINVAL
    assert fill(k=None) == abi.RTP_EINVAL
    assert fill(kr=FAKE + 8) == abi.RTP_EINVAL          # misaligned
    assert fill(n_ring=0) == abi.RTP_OK                 # no-op


def test_noalloc_step_limit_and_rejects():
    """The no-allocation step states its scratch (32 MiB) and rejects sizes beyond it, or
    invalid ones, before any device call."""
    assert abi.rtp_decode_step_noalloc_limit() == 32 << 20
    assert "ESCRATCH" in abi.status_string(abi.RTP_ESCRATCH)
    f = abi.lib().rtp_decode_step_noalloc

    def call(B=1, Hq=8, Hkv=2, n_ret=2, n_loc=6, max_ctx=4096, block=64, split=256, window=64, sinks=4):
        return f(*([FAKE] * 10), 0, B, Hq, Hkv, n_ret, n_loc, max_ctx, block, split, window, sinks,
                 FAKE, FAKE, None, FAKE, None, 0, None, None, 0, None)
    assert call(B=64, Hq=32, Hkv=8, n_ret=32, n_loc=0, max_ctx=1 << 20, block=128, split=128) == abi.RTP_ESCRATCH
    assert call(B=8, Hq=32, Hkv=8, n_ret=16, n_loc=16, max_ctx=1 << 20, block=128, split=128) == abi.RTP_ESCRATCH
    assert call(block=32) == abi.RTP_EUNSUPPORTED
    assert call(split=100) == abi.RTP_EINVAL
    assert call(n_ret=5, n_loc=5) == abi.RTP_EINVAL
    assert call(window=0, sinks=0) == abi.RTP_EINVAL


def test_decode_attn_and_merge_reject():
    L = abi.lib()

    def attn(B=1, Hq=8, Hkv=2, n_ret=2, n_loc=6, block=64, split=1024, window=1024, sinks=4, ws_bytes=1 << 30,
             o=FAKE, loc=FAKE, q=FAKE):
        return L.rtp_decode_attn(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, loc, B, Hq, Hkv, n_ret, n_loc, 4096,
                                 block, split, window, sinks, o, FAKE, FAKE, ws_bytes, None, 0, None, None, 0, None)
    assert attn(B=0) == abi.RTP_EINVAL
    assert attn(n_ret=3) == abi.RTP_EINVAL            # more heads than query heads
    assert attn(Hkv=3) == abi.RTP_EINVAL
    assert attn(block=32) == abi.RTP_EUNSUPPORTED
    assert attn(split=100) == abi.RTP_EINVAL
    assert attn(o=None) == abi.RTP_EINVAL
    assert attn(loc=None) == abi.RTP_EINVAL
    assert attn(window=0, sinks=0) == abi.RTP_EINVAL
    assert attn(ws_bytes=16) == abi.RTP_EINVAL         # local workspace too small
    assert attn(q=FAKE + 8) == abi.RTP_EINVAL          # misaligned
    assert attn(n_ret=0, n_loc=0) == abi.RTP_OK        # nothing to do

    def merge(B=1, n_ret=2, n_loc=6, split=1024, ws_bytes=1 << 30, out=FAKE):
        return L.rtp_decode_merge(FAKE, FAKE, FAKE, FAKE, B, 8, 2, n_ret, n_loc, 4096, split, 1024, 4, FAKE,
                                  ws_bytes, out, None)
    assert merge(B=0) == abi.RTP_EINVAL
    assert merge(out=None) == abi.RTP_EINVAL
    assert merge(split=0) == abi.RTP_EINVAL
    assert merge(ws_bytes=16) == abi.RTP_EINVAL
    assert merge(n_ret=0, n_loc=0) == abi.RTP_OK


def test_probes_reject():
    L = abi.lib()
    F = ctypes.c_void_p(FAKE)
    assert L.rtp_mfma_rate(None, F, 1, 1, None) == 1
    assert L.rtp_mfma_rate(F, None, 1, 1, None) == 1
    assert L.rtp_mfma_rate(ctypes.c_void_p(FAKE + 8), F, 1, 1, None) == 1
    assert L.rtp_mfma_rate(F, F, 0, 1, None) == 1
    assert L.rtp_mfma_rate(F, F, 65536, 1, None) == 1
    assert L.rtp_mfma_rate(F, F, 1, 0, None) == 1
    assert L.rtp_mfma_rate(F, F, 1, 16385, None) == 1
    assert L.rtp_stream_read(F, ctypes.c_size_t(24), F, 1, 1, None) == 1
    assert L.rtp_stream_read(F, ctypes.c_size_t(16), F, 0, 1, None) == 1
