// One decode step as a single host call: the four calls of the path enqueued in order
// from C, so the host pays one call instead of four plus the event calls (the step's
// enqueue cost decides the latency when the device work is short, as at 1M tokens).

#include "rtp_common.hpp"

using rtp::ceil_div;

extern "C" rtp_status rtp_decode_step(
    const void* q_pre, const void* w_q, const void* k_idx, const void* q, const void* k_cache,
    const void* v_cache, const int* seq_lens, const int* ret_heads, const int* loc_heads, const float* top_p,
    int k_tokens, int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx, int block, int split_tokens, int window,
    int sinks, int* sel_idx, int* sel_cnt, unsigned char* sel_mask, float* o_part, float* lse_part, float* out,
    void* ws_index, size_t ws_index_bytes, void* ws_local, size_t ws_local_bytes, const int* kv_slot,
    int n_full, const void* k_ring, const void* v_ring, int n_ring, void* stream, void* side_stream, void* ev_fork,
    void* ev_join) {
  // every argument is checked before anything is enqueued
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_ctx <= 0 || n_ret < 0 || n_loc < 0 || n_ret + n_loc > Hq)
    return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return RTP_EUNSUPPORTED;
  if (!q || !seq_lens || !out) return RTP_EINVAL;
  if (kv_slot) {
    if (n_full < 0 || n_full > Hkv || n_ring < 0 || n_ring > Hkv || n_full + n_ring < 1 ||
        n_full + n_ring > Hkv)
      return RTP_EINVAL;
    if ((n_full > 0 || n_ret > 0) && (!k_cache || !v_cache || n_full < 1)) return RTP_EINVAL;
    if (n_ring > 0 && (!k_ring || !v_ring)) return RTP_EINVAL;
    if (((uintptr_t)k_ring | (uintptr_t)v_ring) & 15) return RTP_EINVAL;
  } else if (!k_cache || !v_cache) {
    return RTP_EINVAL;
  }
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return RTP_EINVAL;
  if (n_ret > 0) {
    if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
    if (split_tokens <= 0 || split_tokens % block) return RTP_EINVAL;
    if (split_tokens / block > 2048 || ceil_div(max_ctx, split_tokens) > 65535) return RTP_EUNSUPPORTED;
    if (k_tokens < 0) return RTP_EINVAL;
    if (!q_pre || !w_q || !k_idx || !ret_heads || (k_tokens == 0 && !top_p) || !sel_idx || !sel_cnt || !o_part ||
        !lse_part || !ws_index)
      return RTP_EINVAL;
    if (((uintptr_t)q_pre | (uintptr_t)w_q | (uintptr_t)k_idx) & 15) return RTP_EINVAL;
    const size_t need = rtp_index_topp_workspace_size(B, n_ret, max_ctx, block);
    if (need == 0) return RTP_EUNSUPPORTED;  // more blocks than one selection holds
    if (ws_index_bytes < need || ((uintptr_t)ws_index & 255)) return RTP_EINVAL;
  }
  if (n_loc > 0) {
    if (window < 0 || sinks < 0 || window + sinks < 1 || !loc_heads || !ws_local) return RTP_EINVAL;
    const size_t need = rtp_local_window_workspace_size(B, Hq, Hkv, n_loc, max_ctx, window, sinks);
    if (need == 0 || ws_local_bytes < need || ((uintptr_t)ws_local & 255)) return RTP_EINVAL;
  }
  const int n_split = n_ret > 0 ? ceil_div(max_ctx, split_tokens) : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fork = n_loc > 0 && n_ret > 0 && side_stream && ev_fork && ev_join;
  rtp_status st = RTP_OK;
  if (n_loc > 0) {
    hipStream_t ls = s;
    if (fork) {
      ls = static_cast<hipStream_t>(side_stream);
      if (hipEventRecord(static_cast<hipEvent_t>(ev_fork), s) != hipSuccess ||
          hipStreamWaitEvent(ls, static_cast<hipEvent_t>(ev_fork), 0) != hipSuccess)
        return RTP_ELAUNCH;
    }
    st = rtp_local_window_attn(q, k_cache, v_cache, seq_lens, loc_heads, B, Hq, Hkv, n_loc, max_ctx, window,
                               sinks, out, ws_local, ws_local_bytes, kv_slot, n_full, k_ring, v_ring, n_ring, ls);
    if (st != RTP_OK) return st;
    if (fork && hipEventRecord(static_cast<hipEvent_t>(ev_join), ls) != hipSuccess) return RTP_ELAUNCH;
  }
  if (n_ret > 0) {
    st = k_tokens > 0 ? rtp_index_topk(q_pre, w_q, k_idx, seq_lens, ret_heads, k_tokens, B, Hq, n_ret, max_ctx,
                                       block, sel_idx, sel_cnt, sel_mask, ws_index, ws_index_bytes, stream)
                      : rtp_index_topp(q_pre, w_q, k_idx, seq_lens, ret_heads, top_p, B, Hq, n_ret, max_ctx, block,
                                       sel_idx, sel_cnt, sel_mask, ws_index, ws_index_bytes, stream);
    if (st == RTP_OK)
      st = rtp_sparse_attn_split(q, k_cache, v_cache, seq_lens, ret_heads, sel_idx, sel_cnt, sel_mask, B, Hq, Hkv,
                                 n_ret, max_ctx, block, split_tokens, o_part, lse_part, kv_slot, n_full, stream);
    if (st == RTP_OK) st = rtp_split_reduce(o_part, lse_part, ret_heads, B, Hq, n_ret, n_split, out, stream);
  }
  if (fork && hipStreamWaitEvent(s, static_cast<hipEvent_t>(ev_join), 0) != hipSuccess) return RTP_ELAUNCH;
  return st;
}
