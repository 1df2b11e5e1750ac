// Decode-side cache maintenance, the step before the path: the decode token's K and V
// rows go into the caches and its low-rank index key k_idx = W^K_h k^pre of every
// retrieval head h into the index-key cache (Review, Adaptive sparse attention
// equation, the key side of s_h(m, n); Review, Method overview: retrieval heads keep
// the full KV cache).  The token is the last of the sequence's N_b tokens (row N_b - 1).
//
// gfx950 launch: one 256-thread workgroup per sequence.  The K/V rows are 16-byte
// copies; each index-key dim is 16 lanes x 8 dims of bf16 products whose exact sum is
// rounded once to bf16, nearest-even (index_key_bf16: an fp64 sum when its error bound
// cannot change the rounding, else an exact integer sum).

#include "rtp_common.hpp"

namespace rtp {
namespace {

constexpr int kAppendThreads = 256;

struct AppendArgs {
  const uint4* k_new;  // bf16 [B, Hkv, 128]
  const uint4* v_new;  // bf16 [B, Hkv, 128]
  const uint16_t* k_pre;  // bf16 [B, Hkv, 128]
  const uint16_t* w_k;    // bf16 [n_ret, 16, 128]
  const int* seq_lens;
  const int* ret_heads;
  int Hq, Hkv, n_ret, max_ctx;
  uint4* kc;           // bf16 [B, n_full, max_ctx, 128]
  uint4* vc;
  uint16_t* kidx;      // bf16 [B, n_ret, max_ctx, 16]
  // KV placement (as the local heads' call reads it): kv_slot[g] >= 0: group g in kc/vc
  // at index kv_slot[g]; < 0: in the sink + window ring kr/vr at index -1 - kv_slot[g]
  // ([B, n_ring, sinks + window, 128]), position p at row p (p < sinks) or
  // sinks + (p - sinks) mod window (a position past the sinks with window 0 is dropped).
  // Null: identity.
  const int* kv_slot;
  uint4* kr;
  uint4* vr;
  int n_full, n_ring, sinks, window;
};

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int pos = a.seq_lens[b] - 1;
  // K and V rows: 16 loads of 16 bytes each per KV head
  for (int i = tid; i < a.Hkv * 32; i += kAppendThreads) {
    const int g = i >> 5, part = i & 31, c = part & 15;
    const uint4 v = (part < 16 ? a.k_new : a.v_new)[((size_t)b * a.Hkv + g) * 16 + c];
    const int slot = a.kv_slot ? a.kv_slot[g] : g;
    if (slot >= 0) {
      (part < 16 ? a.kc : a.vc)[(((size_t)b * a.n_full + slot) * a.max_ctx + pos) * 16 + c] = v;
    } else {
      const int row = pos < a.sinks ? pos : (a.window > 0 ? a.sinks + (pos - a.sinks) % a.window : -1);
      if (row >= 0)
        (part < 16 ? a.kr : a.vr)[(((size_t)b * a.n_ring + (-1 - slot)) * (a.sinks + a.window) + row) * 16 + c] = v;
    }
  }
  // index keys: 16 lanes per (retrieval head, key dim); every pass of the workgroup
  // takes 16 of them, so all lanes of a wave run the same number of passes
  const int G = a.Hq / a.Hkv, part = tid & 15;
  for (int w = tid >> 4; w < a.n_ret * kIndexDim; w += kAppendThreads / 16) {
    const int r = w >> 4, i = w & 15;
    const int kv = a.ret_heads[r] / G;
    const uint4 wv = ld16(a.w_k + ((size_t)r * kIndexDim + i) * kHeadDim + part * 8);
    const uint4 kq = ld16(a.k_pre + ((size_t)b * a.Hkv + kv) * kHeadDim + part * 8);
    const uint32_t key = index_key_bf16(wv, kq);  // the exact sum over the 16 lanes, rounded once
    if (part == 0) a.kidx[(((size_t)b * a.n_ret + r) * a.max_ctx + pos) * kIndexDim + i] = (uint16_t)key;
  }
}

// Ring fill after a prefill: ring row r of a ring group receives the position it holds
// once the prompt's N tokens are in (r < S: position r; r = S + j: the latest position
// p < N with p >= max(S, N - W) and (p - S) mod W = j); rows no position maps to are
// left untouched.  One workgroup per 16 ring rows of a (KV group, sequence): 16 lanes
// copy a 256-byte K row and another 16 its V row.
constexpr int kFillRows = 16;

struct FillArgs {
  const uint4* k;  // bf16 [B, Hkv, T, 128]
  const uint4* v;
  const int* seq_lens;
  const int* kv_slot;
  uint4* kr;       // bf16 [B, n_ring, S + W, 128]
  uint4* vr;
  int Hkv, T, n_ring, sinks, window;
};

__global__ __launch_bounds__(kAppendThreads) void ring_fill_kernel(FillArgs a) {
  const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int slot = a.kv_slot[g];
  if (slot >= 0) return;
  const int N = a.seq_lens[b], S = a.sinks, W = a.window;
  const int r = blockIdx.x * kFillRows + (tid >> 4);  // one ring row per 16 threads
  if (r >= S + W) return;
  int p;
  if (r < S) {
    p = r < N ? r : -1;
  } else {
    const int j = r - S;
    p = N - 1 - ((((N - 1 - S - j) % W) + W) % W);
    if (p < max(S, N - W)) p = -1;
  }
  if (p < 0) return;
  const int c = tid & 15;
  const size_t src = (((size_t)b * a.Hkv + g) * a.T + p) * 16 + c;
  const size_t dst = (((size_t)b * a.n_ring + (-1 - slot)) * (S + W) + r) * 16 + c;
  a.kr[dst] = a.k[src];
  a.vr[dst] = a.v[src];
}

}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" rtp_status rtp_ring_fill(const void* k, const void* v, const int* seq_lens, const int* kv_slot, int B,
                                    int Hkv, int max_ctx, void* k_ring, void* v_ring, int n_ring, int sinks,
                                    int window, void* stream) {
  if (B <= 0 || Hkv <= 0 || max_ctx <= 0 || n_ring < 0 || n_ring > Hkv || sinks < 0 || window < 0) return RTP_EINVAL;
  if (n_ring == 0) return RTP_OK;
  if (sinks + window < 1) return RTP_EINVAL;
  if (!k || !v || !seq_lens || !kv_slot || !k_ring || !v_ring) return RTP_EINVAL;
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_ring | (uintptr_t)v_ring) & 15) return RTP_EINVAL;
  if (B > 65535 || Hkv > 65535) return RTP_EUNSUPPORTED;
  const FillArgs a{static_cast<const uint4*>(k), static_cast<const uint4*>(v), seq_lens, kv_slot,
                   static_cast<uint4*>(k_ring), static_cast<uint4*>(v_ring), Hkv, max_ctx, n_ring, sinks, window};
  hipLaunchKernelGGL(ring_fill_kernel, dim3(ceil_div(sinks + window, kFillRows), Hkv, B), dim3(kAppendThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" rtp_status rtp_cache_append(const void* k_new, const void* v_new, const void* k_pre, const void* w_k,
                                       const int* seq_lens, const int* ret_heads, int B, int Hq, int Hkv, int n_ret,
                                       int max_ctx, void* k_cache, void* v_cache, void* k_idx, const int* kv_slot,
                                       int n_full, void* k_ring, void* v_ring, int n_ring, int sinks, int window,
                                       void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (!k_new || !v_new || !seq_lens) return RTP_EINVAL;
  if (kv_slot) {
    if (n_full < 0 || n_full > Hkv || n_ring < 0 || n_ring > Hkv || n_full + n_ring < 1 ||
        n_full + n_ring > Hkv)
      return RTP_EINVAL;
    if (n_full > 0 && (!k_cache || !v_cache)) return RTP_EINVAL;
    if (n_ring > 0 && (!k_ring || !v_ring || sinks < 0 || window < 0 || sinks + window < 1)) return RTP_EINVAL;
    if (((uintptr_t)k_ring | (uintptr_t)v_ring) & 15) return RTP_EINVAL;
  } else if (!k_cache || !v_cache) {
    return RTP_EINVAL;
  }
  if (n_ret > 0 && (!k_pre || !w_k || !ret_heads || !k_idx)) return RTP_EINVAL;
  if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return RTP_EINVAL;
  if (n_ret > 0 && (((uintptr_t)k_pre | (uintptr_t)w_k) & 15)) return RTP_EINVAL;
  if ((uintptr_t)k_idx & 1) return RTP_EINVAL;
  const AppendArgs a{static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<const uint16_t*>(k_pre), static_cast<const uint16_t*>(w_k), seq_lens, ret_heads,
                     Hq, Hkv, n_ret, max_ctx, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                     static_cast<uint16_t*>(k_idx), kv_slot, static_cast<uint4*>(k_ring), static_cast<uint4*>(v_ring),
                     kv_slot ? n_full : Hkv, kv_slot ? n_ring : 0, sinks, window};
  hipLaunchKernelGGL(append_kernel, dim3(B), dim3(kAppendThreads), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}
