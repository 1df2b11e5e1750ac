// One decode step as a single host call, three launches on the caller's stream: the
// index call (scoring and selection), the attention launch (block-sparse split attention
// of the retrieval heads and window attention of the local heads in one grid) and the
// merge of both kinds of partials.  Only when the local heads' window bytes are large does
// their attention move to a caller-owned second stream, overlapping the index kernel; a
// fork/join of two streams costs tens of microseconds of host time and a few microseconds
// of device time per step, as much as a whole 1M step.

#include <mutex>

#include "rtp_common.hpp"

using rtp::align_up;
using rtp::ceil_div;

namespace {

// Every argument of the step, checked before anything is enqueued.
rtp_status check_step(const void* q_pre, const void* w_q, const void* k_idx, const void* q, const void* k_cache,
                      const void* v_cache, const int* seq_lens, const int* ret_heads, const int* loc_heads,
                      const float* top_p, int k_tokens, int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx,
                      int block, int split_tokens, int window, int sinks, int* sel_idx, int* sel_cnt, float* o_part,
                      float* lse_part, float* out, void* ws_index, size_t ws_index_bytes, void* ws_local,
                      size_t ws_local_bytes, const int* kv_slot, int n_full, const void* k_ring, const void* v_ring,
                      int n_ring) {
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
  return RTP_OK;
}

}  // namespace

extern "C" rtp_status rtp_decode_step(
    const void* q_pre, const void* w_q, const void* k_idx, const void* q, const void* k_cache,
    const void* v_cache, const int* seq_lens, const int* ret_heads, const int* loc_heads, const float* top_p,
    int k_tokens, int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx, int block, int split_tokens, int window,
    int sinks, int* sel_idx, int* sel_cnt, unsigned char* sel_mask, float* o_part, float* lse_part, float* out,
    void* ws_index, size_t ws_index_bytes, void* ws_local, size_t ws_local_bytes, const int* kv_slot,
    int n_full, const void* k_ring, const void* v_ring, int n_ring, void* stream, void* side_stream, void* ev_fork,
    void* ev_join) {
  const rtp_status chk = check_step(q_pre, w_q, k_idx, q, k_cache, v_cache, seq_lens, ret_heads, loc_heads, top_p,
                                    k_tokens, B, Hq, Hkv, n_ret, n_loc, max_ctx, block, split_tokens, window, sinks,
                                    sel_idx, sel_cnt, o_part, lse_part, out, ws_index, ws_index_bytes, ws_local,
                                    ws_local_bytes, kv_slot, n_full, k_ring, v_ring, n_ring);
  if (chk != RTP_OK) return chk;
  // The local heads go to side_stream, overlapping the index kernel, when their window
  // bytes are at least 64 MiB and at least half the index keys' bytes (then they fill the
  // index kernel's selection tail and share its HBM time, and the step is long enough to
  // hide the events' host cost); otherwise everything runs on `stream`, the local heads'
  // workgroups in the attention launch after the split attention's, and no event is
  // recorded (a fork and join cost tens of microseconds of host time).
  const double index_bytes = (double)B * n_ret * max_ctx * 32.0;
  const double local_bytes = (double)B * Hkv * (double)(window + sinks < max_ctx ? window + sinks : max_ctx) * 512.0;
  const bool fork = n_ret > 0 && n_loc > 0 && side_stream && ev_fork && ev_join && 2.0 * local_bytes >= index_bytes &&
                    local_bytes >= 67108864.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rtp_status st = RTP_OK;
  if (fork) {
    hipStream_t ls = static_cast<hipStream_t>(side_stream);
    if (hipEventRecord(static_cast<hipEvent_t>(ev_fork), s) != hipSuccess ||
        hipStreamWaitEvent(ls, static_cast<hipEvent_t>(ev_fork), 0) != hipSuccess)
      return RTP_ELAUNCH;
    st = rtp_decode_attn(q, k_cache, v_cache, seq_lens, nullptr, nullptr, nullptr, nullptr, loc_heads, B, Hq, Hkv, 0,
                         n_loc, max_ctx, block, split_tokens, window, sinks, nullptr, nullptr, ws_local, ws_local_bytes,
                         kv_slot, n_full, k_ring, v_ring, n_ring, ls);
    if (st != RTP_OK) return st;
    if (hipEventRecord(static_cast<hipEvent_t>(ev_join), ls) != hipSuccess) return RTP_ELAUNCH;
  }
  if (n_ret > 0)
    st = k_tokens > 0 ? rtp_index_topk(q_pre, w_q, k_idx, seq_lens, ret_heads, k_tokens, B, Hq, n_ret, max_ctx,
                                       block, sel_idx, sel_cnt, sel_mask, ws_index, ws_index_bytes, stream)
                      : rtp_index_topp(q_pre, w_q, k_idx, seq_lens, ret_heads, top_p, B, Hq, n_ret, max_ctx, block,
                                       sel_idx, sel_cnt, sel_mask, ws_index, ws_index_bytes, stream);
  if (st == RTP_OK)
    st = rtp_decode_attn(q, k_cache, v_cache, seq_lens, ret_heads, sel_idx, sel_cnt, sel_mask, loc_heads, B, Hq, Hkv,
                         n_ret, fork ? 0 : n_loc, max_ctx, block, split_tokens, window, sinks, o_part, lse_part,
                         ws_local, ws_local_bytes, kv_slot, n_full, k_ring, v_ring, n_ring, stream);
  if (fork && hipStreamWaitEvent(s, static_cast<hipEvent_t>(ev_join), 0) != hipSuccess) return RTP_ELAUNCH;
  if (st == RTP_OK)
    st = rtp_decode_merge(o_part, lse_part, ret_heads, loc_heads, B, Hq, Hkv, n_ret, n_loc, max_ctx, split_tokens,
                          window, sinks, ws_local, ws_local_bytes, out, stream);
  return st;
}

// ---------------------------------------------------------------- no-allocation step
// The same step for callers that cannot allocate (code under HIP graph capture, tight
// serving loops): the index and local workspaces and the split partials live in one
// file-scope device array.  Host code never passes the array's name to a kernel (there it
// is a host-side stand-in); the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {

constexpr size_t kScratchIndexBytes = 16u << 20;  // index workspace (per-head state)
constexpr size_t kScratchLocalBytes = 8u << 20;   // local heads' window partials
constexpr size_t kScratchPartBytes = 8u << 20;    // split partials (o, then lse)
constexpr size_t kScratchBytes = kScratchIndexBytes + kScratchLocalBytes + kScratchPartBytes;
constexpr int kScratchDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchState {
  char* ptr = nullptr;  // this device's copy of `scratch`
  int nblk = -1;        // blocks per sequence the index region was cleared for
};
std::mutex g_scratch_mu;
ScratchState g_scratch[kScratchDevices];

constexpr int kClearThreads = 256;

__global__ __launch_bounds__(kClearThreads) void clear_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * kClearThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * kClearThreads)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" size_t rtp_decode_step_noalloc_limit(void) { return kScratchBytes; }

extern "C" rtp_status rtp_decode_step_noalloc(
    const void* q_pre, const void* w_q, const void* k_idx, const void* q, const void* k_cache,
    const void* v_cache, const int* seq_lens, const int* ret_heads, const int* loc_heads, const float* top_p,
    int k_tokens, int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx, int block, int split_tokens, int window,
    int sinks, int* sel_idx, int* sel_cnt, unsigned char* sel_mask, float* out, const int* kv_slot, int n_full,
    const void* k_ring, const void* v_ring, int n_ring, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_ctx <= 0 || n_ret < 0 || n_loc < 0 || n_ret + n_loc > Hq)
    return RTP_EINVAL;
  // the scratch each part needs, against its share of the array
  size_t ws_index = 0, ws_local = 0, part = 0;
  int n_split = 0, nblk = 0;
  if (n_ret > 0) {
    if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
    if (split_tokens <= 0 || split_tokens % block) return RTP_EINVAL;
    ws_index = rtp_index_topp_workspace_size(B, n_ret, max_ctx, block);
    if (ws_index == 0) return RTP_EUNSUPPORTED;
    n_split = ceil_div(max_ctx, split_tokens);
    nblk = ceil_div(max_ctx, block);
    part = align_up((size_t)B * n_ret * n_split * RTP_HEAD_DIM * sizeof(float), 256) +
           (size_t)B * n_ret * n_split * sizeof(float);
  }
  if (n_loc > 0) {
    ws_local = rtp_local_window_workspace_size(B, Hq, Hkv, n_loc, max_ctx, window, sinks);
    if (ws_local == 0) return RTP_EINVAL;
  }
  if (ws_index > kScratchIndexBytes || ws_local > kScratchLocalBytes || part > kScratchPartBytes)
    return RTP_ESCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return RTP_ELAUNCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchState& st = g_scratch[dev];
    if (!st.ptr) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RTP_ELAUNCH;
      st.ptr = static_cast<char*>(p);
    }
    base = st.ptr;
    const size_t o_bytes = align_up((size_t)B * n_ret * n_split * RTP_HEAD_DIM * sizeof(float), 256);
    float* o_chk = reinterpret_cast<float*>(base + kScratchIndexBytes + kScratchLocalBytes);
    const rtp_status chk =
        check_step(q_pre, w_q, k_idx, q, k_cache, v_cache, seq_lens, ret_heads, loc_heads, top_p, k_tokens, B, Hq,
                   Hkv, n_ret, n_loc, max_ctx, block, split_tokens, window, sinks, sel_idx, sel_cnt, o_chk,
                   reinterpret_cast<float*>(reinterpret_cast<char*>(o_chk) + o_bytes), out, base, kScratchIndexBytes,
                   base + kScratchIndexBytes, kScratchLocalBytes, kv_slot, n_full, k_ring, v_ring, n_ring);
    if (chk != RTP_OK) return chk;
    // the index region starts zero-filled for each number of blocks per sequence (its
    // per-head state is laid out by it); a fill kernel, so graph capture records no memset
    if (n_ret > 0 && st.nblk != nblk) {
      hipLaunchKernelGGL(clear_kernel, dim3(1024), dim3(kClearThreads), 0, s, reinterpret_cast<uint4*>(base),
                         kScratchIndexBytes / 16);
      if (hipGetLastError() != hipSuccess) return RTP_ELAUNCH;
      st.nblk = nblk;
    }
  }
  char* idx_ws = base;
  char* loc_ws = base + kScratchIndexBytes;
  float* o_part = reinterpret_cast<float*>(base + kScratchIndexBytes + kScratchLocalBytes);
  float* lse_part = reinterpret_cast<float*>(reinterpret_cast<char*>(o_part) +
                                             align_up((size_t)B * n_ret * n_split * RTP_HEAD_DIM * sizeof(float), 256));
  return rtp_decode_step(q_pre, w_q, k_idx, q, k_cache, v_cache, seq_lens, ret_heads, loc_heads, top_p, k_tokens, B,
                         Hq, Hkv, n_ret, n_loc, max_ctx, block, split_tokens, window, sinks, sel_idx, sel_cnt,
                         sel_mask, n_ret > 0 ? o_part : nullptr, n_ret > 0 ? lse_part : nullptr, out,
                         n_ret > 0 ? idx_ws : nullptr, ws_index, n_loc > 0 ? loc_ws : nullptr, ws_local, kv_slot,
                         n_full, k_ring, v_ring, n_ring, stream, nullptr, nullptr, nullptr);
}
