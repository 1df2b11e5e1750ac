"""Thin ctypes binding of librtp.so (see include/rtp.h).

Argument marshalling only: every function passes raw device pointers, sizes and
the current HIP stream to the C ABI of the same name and raises on a non-zero
status.  PyTorch provides device memory and streams; all computation runs in the
HIP kernels of librtp.so.  A missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librtp.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rtp.h")

RTP_OK, RTP_EINVAL, RTP_EUNSUPPORTED, RTP_ELAUNCH, RTP_ESCRATCH = 0, 1, 2, 3, 4

_lib = None


class RTPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "rtp_status_string": ([_i], ctypes.c_char_p),
    "rtp_version": ([], ctypes.c_char_p),
    "rtp_index_topp_workspace_size": ([_i, _i, _i, _i], _sz),
    "rtp_index_topp": ([_vp] * 6 + [_i] * 5 + [_vp, _vp, _vp, _vp, _sz, _vp], _i),
    "rtp_index_topk": ([_vp] * 5 + [_i] * 6 + [_vp, _vp, _vp, _vp, _sz, _vp], _i),
    "rtp_sparse_attn_split": ([_vp] * 8 + [_i] * 7 + [_vp, _vp, _vp, _i, _vp], _i),
    "rtp_split_reduce": ([_vp] * 3 + [_i] * 4 + [_vp, _vp], _i),
    "rtp_local_window_workspace_size": ([_i] * 7, _sz),
    "rtp_local_window_attn": ([_vp] * 5 + [_i] * 7 + [_vp, _vp, _sz, _vp, _i, _vp, _vp, _i, _vp], _i),
    "rtp_decode_step": ([_vp] * 10 + [_i] * 11 + [_vp] * 6 + [_vp, _sz, _vp, _sz] + [_vp, _i, _vp, _vp, _i]
                        + [_vp] * 4, _i),
    "rtp_decode_attn": ([_vp] * 9 + [_i] * 10 + [_vp] * 3 + [_sz, _vp, _i, _vp, _vp, _i, _vp], _i),
    "rtp_decode_merge": ([_vp] * 4 + [_i] * 9 + [_vp, _sz, _vp, _vp], _i),
    "rtp_decode_step_noalloc_limit": ([], _sz),
    "rtp_decode_step_noalloc": ([_vp] * 10 + [_i] * 11 + [_vp] * 4 + [_vp, _i, _vp, _vp, _i] + [_vp], _i),
    "rtp_stream_read": ([_vp, _sz, _vp, _i, _i, _vp], _i),
    "rtp_mfma_rate": ([_vp, _vp, _i, _i, _vp], _i),
    "rtp_cache_append": ([_vp] * 6 + [_i] * 5 + [_vp] * 3 + [_vp, _i, _vp, _vp, _i, _i, _i, _vp], _i),
    "rtp_prefill_attn": ([_vp] * 5 + [_i] * 7 + [_vp, _vp], _i),
    "rtp_prefill_index_keys": ([_vp] * 4 + [_i] * 5 + [_vp, _vp], _i),
    "rtp_ring_fill": ([_vp] * 4 + [_i] * 3 + [_vp, _vp] + [_i] * 3 + [_vp], _i),
}


def lib() -> ctypes.CDLL:
    """Load librtp.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_sparse_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions include/rtp.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rtp_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().rtp_status_string(int(status)).decode()


def version() -> str:
    return lib().rtp_version().decode()


def device_ptr(t: torch.Tensor) -> int:
    """Raw device address of a contiguous device tensor (raises otherwise)."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("librtp arguments must be contiguous device tensors")
    return t.data_ptr()


def nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def check(fn: str, st: int) -> None:
    if st != RTP_OK:
        raise RTPError(fn, st)


# ---- HIP events for ordering the step's two streams (plumbing only)
_hip = None


def _hip_lib() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        lib()  # librtp.so links the HIP runtime; load the same copy
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventCreateWithFlags.restype = ctypes.c_int
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventRecord.restype = ctypes.c_int
        h.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        h.hipStreamWaitEvent.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        _hip = h
    return _hip


# Flags of the events that order the step's two streams on one device: no timing
# (hipEventDisableTiming) and no system-scope fence at the record
# (hipEventDisableSystemFence), which only the host or other devices would need; the
# producer's writes stay visible to the other stream's kernels on the same device.
EVENT_DEVICE_ORDER = 0x2 | 0x20000000


def event_create(flags: int = 0x2) -> int:
    """A HIP event (default: hipEventDisableTiming)."""
    ev = ctypes.c_void_p()
    st = _hip_lib().hipEventCreateWithFlags(ctypes.byref(ev), flags)
    if st != 0:
        raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
    return ev.value


def event_record(ev: int, stream: int) -> None:
    st = _hip.hipEventRecord(ev, stream)
    if st != 0:
        raise RuntimeError(f"hipEventRecord failed ({st})")


def stream_wait_event(stream: int, ev: int) -> None:
    st = _hip.hipStreamWaitEvent(stream, ev, 0)
    if st != 0:
        raise RuntimeError(f"hipStreamWaitEvent failed ({st})")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else device_ptr(t)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _s(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_check = check


def rtp_index_topp_workspace_size(B: int, n_ret: int, max_ctx: int, block: int) -> int:
    return int(lib().rtp_index_topp_workspace_size(B, n_ret, max_ctx, block))


def rtp_local_window_workspace_size(B: int, Hq: int, Hkv: int, n_loc: int, max_ctx: int,
                                    window: int, sinks: int) -> int:
    return int(lib().rtp_local_window_workspace_size(B, Hq, Hkv, n_loc, max_ctx, window, sinks))


def rtp_index_topp(q_pre, w_q, k_idx, seq_lens, ret_heads, top_p, B, Hq, n_ret, max_ctx, block,
                   sel_idx, sel_cnt, workspace, stream=None, sel_mask=None) -> None:
    st = lib().rtp_index_topp(_p(q_pre), _p(w_q), _p(k_idx), _p(seq_lens), _p(ret_heads), _p(top_p),
                              B, Hq, n_ret, max_ctx, block, _p(sel_idx), _p(sel_cnt), _p(sel_mask), _p(workspace),
                              _nbytes(workspace), _s(stream))
    _check("rtp_index_topp", st)


def rtp_index_topk(q_pre, w_q, k_idx, seq_lens, ret_heads, k_tokens, B, Hq, n_ret, max_ctx, block,
                   sel_idx, sel_cnt, workspace, stream=None, sel_mask=None) -> None:
    st = lib().rtp_index_topk(_p(q_pre), _p(w_q), _p(k_idx), _p(seq_lens), _p(ret_heads), int(k_tokens),
                              B, Hq, n_ret, max_ctx, block, _p(sel_idx), _p(sel_cnt), _p(sel_mask), _p(workspace),
                              _nbytes(workspace), _s(stream))
    _check("rtp_index_topk", st)


def rtp_sparse_attn_split(q, k_cache, v_cache, seq_lens, ret_heads, sel_idx, sel_cnt, B, Hq, Hkv,
                          n_ret, max_ctx, block, split_tokens, o_part, lse_part, stream=None, sel_mask=None,
                          kv_slot=None, n_full=0) -> None:
    st = lib().rtp_sparse_attn_split(_p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(ret_heads),
                                     _p(sel_idx), _p(sel_cnt), _p(sel_mask), B, Hq, Hkv, n_ret, max_ctx, block,
                                     split_tokens, _p(o_part), _p(lse_part), _p(kv_slot), n_full, _s(stream))
    _check("rtp_sparse_attn_split", st)


def rtp_decode_step_noalloc_limit() -> int:
    return int(lib().rtp_decode_step_noalloc_limit())


def rtp_decode_step_noalloc(q_pre, w_q, k_idx, q, k_cache, v_cache, seq_lens, ret_heads, loc_heads, top_p, k_tokens,
                            B, Hq, Hkv, n_ret, n_loc, max_ctx, block, split_tokens, window, sinks,
                            sel_idx, sel_cnt, sel_mask, out, stream=None, kv_slot=None, n_full=0, k_ring=None,
                            v_ring=None, n_ring=0) -> None:
    """rtp_decode_step with its workspaces and partials in the library's fixed device scratch."""
    st = lib().rtp_decode_step_noalloc(_p(q_pre), _p(w_q), _p(k_idx), _p(q), _p(k_cache), _p(v_cache),
                                       _p(seq_lens), _p(ret_heads), _p(loc_heads), _p(top_p), int(k_tokens), B, Hq,
                                       Hkv, n_ret, n_loc, max_ctx, block, split_tokens, window, sinks, _p(sel_idx),
                                       _p(sel_cnt), _p(sel_mask), _p(out), _p(kv_slot), n_full, _p(k_ring),
                                       _p(v_ring), n_ring, _s(stream))
    _check("rtp_decode_step_noalloc", st)


def rtp_decode_attn(q, k_cache, v_cache, seq_lens, ret_heads, sel_idx, sel_cnt, sel_mask, loc_heads, B, Hq, Hkv,
                    n_ret, n_loc, max_ctx, block, split_tokens, window, sinks, o_part, lse_part, ws_local,
                    stream=None, kv_slot=None, n_full=0, k_ring=None, v_ring=None, n_ring=0) -> None:
    st = lib().rtp_decode_attn(_p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(ret_heads), _p(sel_idx),
                               _p(sel_cnt), _p(sel_mask), _p(loc_heads), B, Hq, Hkv, n_ret, n_loc, max_ctx, block,
                               split_tokens, window, sinks, _p(o_part), _p(lse_part), _p(ws_local), _nbytes(ws_local),
                               _p(kv_slot), n_full, _p(k_ring), _p(v_ring), n_ring, _s(stream))
    _check("rtp_decode_attn", st)


def rtp_decode_merge(o_part, lse_part, ret_heads, loc_heads, B, Hq, Hkv, n_ret, n_loc, max_ctx, split_tokens, window,
                     sinks, ws_local, out, stream=None) -> None:
    st = lib().rtp_decode_merge(_p(o_part), _p(lse_part), _p(ret_heads), _p(loc_heads), B, Hq, Hkv, n_ret, n_loc,
                                max_ctx, split_tokens, window, sinks, _p(ws_local), _nbytes(ws_local), _p(out),
                                _s(stream))
    _check("rtp_decode_merge", st)


def rtp_stream_read(src, sink, n_workgroups: int, nontemporal: bool = True, stream=None) -> None:
    """Calibration probe: one read-only pass over `src` (see rtp.h)."""
    st = lib().rtp_stream_read(_p(src), _nbytes(src), _p(sink), int(n_workgroups), int(bool(nontemporal)),
                               _s(stream))
    _check("rtp_stream_read", st)


def rtp_mfma_rate(ops, out, n_workgroups: int, iters: int, stream=None) -> None:
    """Calibration probe: back-to-back bf16 MFMAs (see rtp.h); `ops` bf16 [2, 64, 8], `out`
    holds n_workgroups * 256 fp32."""
    if ops.numel() * ops.element_size() < 2048 or out.numel() < int(n_workgroups) * 256:
        raise ValueError("rtp_mfma_rate: ops needs 2 x 64 x 8 bf16 and out n_workgroups * 256 values")
    st = lib().rtp_mfma_rate(_p(ops), _p(out), int(n_workgroups), int(iters), _s(stream))
    _check("rtp_mfma_rate", st)


def rtp_cache_append(k_new, v_new, k_pre, w_k, seq_lens, ret_heads, B, Hq, Hkv, n_ret, max_ctx,
                     k_cache, v_cache, k_idx, stream=None, kv_slot=None, n_full=0, k_ring=None, v_ring=None,
                     n_ring=0, sinks=0, window=0) -> None:
    st = lib().rtp_cache_append(_p(k_new), _p(v_new), _p(k_pre), _p(w_k), _p(seq_lens), _p(ret_heads), B, Hq,
                                Hkv, n_ret, max_ctx, _p(k_cache), _p(v_cache), _p(k_idx), _p(kv_slot), n_full,
                                _p(k_ring), _p(v_ring), n_ring, sinks, window, _s(stream))
    _check("rtp_cache_append", st)


def rtp_split_reduce(o_part, lse_part, heads, B, Hq, n_heads, n_split, out, stream=None) -> None:
    st = lib().rtp_split_reduce(_p(o_part), _p(lse_part), _p(heads), B, Hq, n_heads, n_split, _p(out),
                                _s(stream))
    _check("rtp_split_reduce", st)


def rtp_local_window_attn(q, k_cache, v_cache, seq_lens, loc_heads, B, Hq, Hkv, n_loc, max_ctx,
                          window, sinks, out, workspace, stream=None, kv_slot=None, n_full=0, k_ring=None,
                          v_ring=None, n_ring=0) -> None:
    st = lib().rtp_local_window_attn(_p(q), _p(k_cache), _p(v_cache), _p(seq_lens), _p(loc_heads), B, Hq,
                                     Hkv, n_loc, max_ctx, window, sinks, _p(out), _p(workspace),
                                     _nbytes(workspace), _p(kv_slot), n_full, _p(k_ring), _p(v_ring), n_ring,
                                     _s(stream))
    _check("rtp_local_window_attn", st)


def rtp_prefill_attn(q, k, v, seq_lens, ret_heads, B, Hq, Hkv, n_ret, max_ctx, window, sinks, out,
                     stream=None) -> None:
    st = lib().rtp_prefill_attn(_p(q), _p(k), _p(v), _p(seq_lens), _p(ret_heads) if n_ret else None, B, Hq, Hkv,
                                n_ret, max_ctx, window, sinks, _p(out), _s(stream))
    _check("rtp_prefill_attn", st)


def rtp_prefill_index_keys(k_pre, w_k, seq_lens, ret_heads, B, Hq, Hkv, n_ret, max_ctx, k_idx, stream=None) -> None:
    st = lib().rtp_prefill_index_keys(_p(k_pre), _p(w_k), _p(seq_lens), _p(ret_heads), B, Hq, Hkv, n_ret, max_ctx,
                                      _p(k_idx), _s(stream))
    _check("rtp_prefill_index_keys", st)


def rtp_ring_fill(k, v, seq_lens, kv_slot, B, Hkv, max_ctx, k_ring, v_ring, n_ring, sinks, window,
                  stream=None) -> None:
    st = lib().rtp_ring_fill(_p(k), _p(v), _p(seq_lens), _p(kv_slot), B, Hkv, max_ctx, _p(k_ring), _p(v_ring),
                             n_ring, sinks, window, _s(stream))
    _check("rtp_ring_fill", st)
