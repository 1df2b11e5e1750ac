// Kernel 2 of the decode path, the local heads' kernel and the log-sum-exp merge, as
// launches (their attention device code and its description are in rtp_sparse.hpp).
//
// Kernel 2: grid (split, KV group rank), 256 threads; each workgroup writes per-head
// (o, lse) partials of its split, which rtp_split_reduce merges.  KV groups are ranked
// by their selected-block counts, heaviest first, so the grid drains on light work.  Local heads: grid
// (window split, KV group, sequence); the partials go to the workspace and the merge
// kernel (one workgroup per output row, the same kernel as the cross-split reduce)
// combines them with the log-sum-exp rule on the same stream.

#include "rtp_sparse.hpp"

namespace rtp {
namespace {

constexpr int kThreads = kAttnThreads;

template <int BK, int G>
__global__ __launch_bounds__(kThreads) void sparse_attn_kernel(SparseArgs a, int n_split, float* __restrict__ o_part,
                                                               float* __restrict__ lse_part) {
  __shared__ SparseSmem<G> S;
  // workgroups are dispatched in blockIdx order: (split, group rank), heaviest group first
  const int c = blockIdx.x;
  const SparseGroup<G> grp = sparse_group<G>(a, gridDim.z, blockIdx.y + a.Hkv * blockIdx.z, &S);
  const int b = grp.b;
  const int n_ret = a.n_ret;
  sparse_split<BK, G>(a, c, grp, &S, [&](int i, int d, float o, float lse) {
    const size_t hr = (size_t)b * n_ret + i;
    o_part[(hr * n_split + c) * kHeadDim + d] = o;
    if (d == 0) lse_part[hr * n_split + c] = lse;
  });
}

template <int G>
__global__ __launch_bounds__(kThreads) void local_window_kernel(LocalArgs a, int n_split, float* __restrict__ ws_o,
                                                                float* __restrict__ ws_lse) {
  __shared__ LocalSmem<G> S;
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n_loc = a.n_loc;
  local_split<G>(a, c, g, b, &S, [&](int i, int d, float o, float lse) {
    const size_t hr = (size_t)b * n_loc + i;
    ws_o[(hr * n_split + c) * kHeadDim + d] = o;
    if (d == 0) ws_lse[hr * n_split + c] = lse;
  });
}

// Log-sum-exp merge of n_split partials for one output row per workgroup:
// L = log sum_c exp(lse_c); out = sum_c exp(lse_c - L) o_c.  1024 threads = 8 groups of
// 128 (one thread per output dim); group k takes splits k, k + 8, ...  Each thread
// issues the loads of its partial values and their LSEs before the row maximum is
// reduced, kMergeBatch splits at a time, so one memory round trip serves up to 128
// splits; the eight group sums are added in a fixed order.  A row whose partials are
// all empty (lse = -inf) is written 0.
constexpr int kMergeThreads = 1024;
constexpr int kMergeGroups = kMergeThreads / kHeadDim;
constexpr int kMergeBatch = 16;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, const int* __restrict__ heads,
    int Hq, int n_heads, int n_split, float* __restrict__ out) {
  const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = tid & (kHeadDim - 1), grp = tid / kHeadDim;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t hr = (size_t)b * n_heads + i;
  const float* lp = lse_part + hr * n_split;
  const float* op = o_part + hr * n_split * kHeadDim + d;
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ float s_L[kMergeGroups], s_A[kMergeGroups][kHeadDim];
  // this thread's first batch of partials, in flight while the maximum is reduced
  float ov[kMergeBatch], lv[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const int c = grp + u * kMergeGroups;
    ov[u] = c < n_split ? op[(size_t)c * kHeadDim] : 0.f;
    lv[u] = c < n_split ? lp[c] : -INFINITY;
  }
  float mloc = -INFINITY;
  for (int c = tid; c < n_split; c += kMergeThreads) mloc = fmaxf(mloc, lp[c]);
  mloc = wave_maxf(mloc);
  if (lane == 0) s_red[wave] = mloc;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w]);
  float L = 0.f, A = 0.f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < n_split; c0 += kMergeBatch * kMergeGroups) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const int c = c0 + grp + u * kMergeGroups;
          ov[u] = c < n_split ? op[(size_t)c * kHeadDim] : 0.f;
          lv[u] = c < n_split ? lp[c] : -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = __expf(lv[u] - M);  // 0 for empty or absent splits
        L += w;
        A = fmaf(w, ov[u], A);
      }
    }
  }
  if (d == 0) s_L[grp] = L;
  s_A[grp][d] = A;
  __syncthreads();
  if (grp == 0) {
    float Lt = s_L[0], At = s_A[0][d];
#pragma unroll
    for (int k = 1; k < kMergeGroups; ++k) {
      Lt += s_L[k];
      At += s_A[k][d];
    }
    out[((size_t)b * Hq + heads[i]) * kHeadDim + d] = Lt > 0.f ? At / Lt : 0.f;
  }
}

struct LocalLayout {
  int split_tokens, n_split;
  size_t off_lse, off_o, total;
};

LocalLayout local_layout(int B, int Hkv, int n_loc, int window) {
  LocalLayout L{};
  L.split_tokens = local_split_tokens(B, Hkv, window);
  L.n_split = 1 + ceil_div(window, L.split_tokens);
  L.off_lse = 0;
  L.off_o = align_up((size_t)B * n_loc * L.n_split * sizeof(float), 256);
  L.total = L.off_o + align_up((size_t)B * n_loc * L.n_split * kHeadDim * sizeof(float), 256);
  return L;
}

inline bool group_ok(int Hq, int Hkv) {
  if (Hkv <= 0 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

template <int BK>
void launch_sparse(int G, dim3 grid, hipStream_t s, const SparseArgs& a, int n_split, float* op, float* lp) {
#define RTP_SPARSE(GG) \
  hipLaunchKernelGGL((sparse_attn_kernel<BK, GG>), grid, dim3(kThreads), 0, s, a, n_split, op, lp)
  switch (G) {
    case 1: RTP_SPARSE(1); break;
    case 2: RTP_SPARSE(2); break;
    case 4: RTP_SPARSE(4); break;
    default: RTP_SPARSE(8); break;
  }
#undef RTP_SPARSE
}

}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" rtp_status rtp_sparse_attn_split(const void* q, const void* k_cache, const void* v_cache,
                                            const int* seq_lens, const int* ret_heads,
                                            const int* sel_idx, const int* sel_cnt,
                                            const unsigned char* sel_mask, int B, int Hq,
                                            int Hkv, int n_ret, int max_ctx, int block,
                                            int split_tokens, float* o_part, float* lse_part,
                                            const int* kv_slot, int n_full, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (!group_ok(Hq, Hkv)) return RTP_EUNSUPPORTED;
  if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
  if (split_tokens <= 0 || split_tokens % block) return RTP_EINVAL;
  if (split_tokens / block > kMaxSplitBlocks) return RTP_EUNSUPPORTED;
  if (n_ret == 0) return RTP_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !ret_heads || !o_part || !lse_part) return RTP_EINVAL;
  if (!sel_mask && (!sel_idx || !sel_cnt)) return RTP_EINVAL;
  if (kv_slot && (n_full <= 0 || n_full > Hkv)) return RTP_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return RTP_EINVAL;
  const int nblk_max = ceil_div(max_ctx, block);
  const int sb = split_tokens / block;
  const int n_split = ceil_div(max_ctx, split_tokens);
  if (n_split > 65535) return RTP_EUNSUPPORTED;
  dim3 grid(n_split, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const SparseArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), seq_lens, ret_heads, sel_idx, sel_cnt, sel_mask, kv_slot,
                     Hq, Hkv, n_ret, max_ctx, nblk_max, sb, kv_slot ? n_full : Hkv};
  const int G = Hq / Hkv;
  if (block == 64)
    launch_sparse<64>(G, grid, s, a, n_split, o_part, lse_part);
  else
    launch_sparse<128>(G, grid, s, a, n_split, o_part, lse_part);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" rtp_status rtp_split_reduce(const float* o_part, const float* lse_part, const int* heads,
                                       int B, int Hq, int n_heads, int n_split, float* out,
                                       void* stream) {
  if (B <= 0 || Hq <= 0 || n_heads < 0 || n_heads > Hq || n_split <= 0) return RTP_EINVAL;
  if (n_heads == 0) return RTP_OK;
  if (!o_part || !lse_part || !heads || !out) return RTP_EINVAL;
  if (B > 65535) return RTP_EUNSUPPORTED;
  hipLaunchKernelGGL(merge_kernel, dim3(n_heads, B), dim3(kMergeThreads), 0,
                     static_cast<hipStream_t>(stream), o_part, lse_part, heads, Hq, n_heads, n_split,
                     out);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" size_t rtp_local_window_workspace_size(int B, int Hq, int Hkv, int n_loc, int max_ctx,
                                                  int window, int sinks) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_loc <= 0 || n_loc > Hq || max_ctx <= 0 || window < 0 ||
      sinks < 0 || window + sinks < 1 || Hq % Hkv)
    return 0;
  return local_layout(B, Hkv, n_loc, window < max_ctx ? window : max_ctx).total;
}

extern "C" rtp_status rtp_local_window_attn(const void* q, const void* k_cache, const void* v_cache,
                                            const int* seq_lens, const int* loc_heads, int B, int Hq,
                                            int Hkv, int n_loc, int max_ctx, int window, int sinks,
                                            float* out, void* workspace, size_t ws_bytes,
                                            const int* kv_slot, int n_full, const void* k_ring,
                                            const void* v_ring, int n_ring, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_loc < 0 || n_loc > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv || window < 0 || sinks < 0 || window + sinks < 1) return RTP_EINVAL;
  if (!group_ok(Hq, Hkv)) return RTP_EUNSUPPORTED;
  if (n_loc == 0) return RTP_OK;
  if (!q || !seq_lens || !loc_heads || !out || !workspace) return RTP_EINVAL;
  if (kv_slot) {
    // full caches may be absent when every group is in the ring, and the reverse
    if (n_full < 0 || n_full > Hkv || n_ring < 0 || n_ring > Hkv || n_full + n_ring < 1 ||
        n_full + n_ring > Hkv)
      return RTP_EINVAL;
    if (n_full > 0 && (!k_cache || !v_cache)) return RTP_EINVAL;
    if (n_ring > 0 && (!k_ring || !v_ring)) return RTP_EINVAL;
    if (((uintptr_t)k_ring | (uintptr_t)v_ring) & 15) return RTP_EINVAL;
  } else if (!k_cache || !v_cache) {
    return RTP_EINVAL;
  }
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return RTP_EINVAL;
  if ((uintptr_t)workspace & 255) return RTP_EINVAL;
  const LocalLayout L = local_layout(B, Hkv, n_loc, window < max_ctx ? window : max_ctx);
  if (ws_bytes < L.total) return RTP_EINVAL;
  if (L.n_split > 65535) return RTP_EUNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  float* ws_lse = reinterpret_cast<float*>(ws + L.off_lse);
  float* ws_o = reinterpret_cast<float*>(ws + L.off_o);
  dim3 grid(L.n_split, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LocalArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                    static_cast<const uint16_t*>(v_cache), seq_lens, loc_heads, Hq, Hkv, n_loc, max_ctx,
                    window, sinks, L.split_tokens, kv_slot, static_cast<const uint16_t*>(k_ring),
                    static_cast<const uint16_t*>(v_ring), kv_slot ? n_full : Hkv, kv_slot ? n_ring : 0};
#define RTP_LOCAL(GG) \
  hipLaunchKernelGGL(local_window_kernel<GG>, grid, dim3(kThreads), 0, s, a, L.n_split, ws_o, ws_lse)
  switch (Hq / Hkv) {
    case 1: RTP_LOCAL(1); break;
    case 2: RTP_LOCAL(2); break;
    case 4: RTP_LOCAL(4); break;
    default: RTP_LOCAL(8); break;
  }
  hipLaunchKernelGGL(merge_kernel, dim3(n_loc, B), dim3(kMergeThreads), 0, s, ws_o, ws_lse, loc_heads, Hq,
                     n_loc, L.n_split, out);
#undef RTP_LOCAL
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" const char* rtp_status_string(int status) {
  switch (status) {
    case RTP_OK: return "RTP_OK";
    case RTP_EINVAL: return "RTP_EINVAL: invalid argument";
    case RTP_EUNSUPPORTED: return "RTP_EUNSUPPORTED: size outside the supported set";
    case RTP_ELAUNCH: return "RTP_ELAUNCH: kernel launch failed";
    case RTP_ESCRATCH: return "RTP_ESCRATCH: sizes beyond the no-allocation entry point's fixed scratch";
    default: return "RTP_UNKNOWN";
  }
}

extern "C" const char* rtp_version(void) { return "rtp 1.0 gfx950"; }
