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

// Row i of sequence b: n_split partials (o, lse) of partial row (b, i) of an [B, n_rows, n_split]
// set, merged into out[b, head].
__device__ __forceinline__ void merge_row(const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                          int n_rows, int i, int b, int n_split, int head, int Hq,
                                          float* __restrict__ out) {
  const int tid = threadIdx.x;
  const int d = tid & (kHeadDim - 1), grp = tid / kHeadDim;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t hr = (size_t)b * n_rows + i;
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
    out[((size_t)b * Hq + head) * kHeadDim + d] = Lt > 0.f ? At / Lt : 0.f;
  }
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, const int* __restrict__ heads,
    int Hq, int n_heads, int n_split, float* __restrict__ out) {
  const int i = blockIdx.x, b = blockIdx.y;
  merge_row(o_part, lse_part, n_heads, i, b, n_split, heads[i], Hq, out);
}

// The decode step's merge: rows [0, n_ret) of each sequence from the retrieval heads' split
// partials, rows [n_ret, n_ret + n_loc) from the local heads' window partials, one launch.
__global__ __launch_bounds__(kMergeThreads) void merge_step_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, const int* __restrict__ ret_heads,
    int n_ret, int n_split, const float* __restrict__ lo_part, const float* __restrict__ llse_part,
    const int* __restrict__ loc_heads, int n_loc, int n_split_loc, int Hq, float* __restrict__ out) {
  const int i = blockIdx.x, b = blockIdx.y;
  if (i < n_ret)
    merge_row(o_part, lse_part, n_ret, i, b, n_split, ret_heads[i], Hq, out);
  else
    merge_row(lo_part, llse_part, n_loc, i - n_ret, b, n_split_loc, loc_heads[i - n_ret], Hq, out);
}

// The decode step's attention launch: kernel 2's workgroups (split, KV group rank, heaviest
// group first) followed by the local heads' window workgroups (window split, KV group,
// sequence) in one grid; the local workgroups, dispatched last, fill the compute units
// that kernel 2's drain leaves idle.  Both roles write partials for the step's merge.
template <int BK, int G>
__global__ __launch_bounds__(kThreads) void step_attn_kernel(SparseArgs a, int B, int n_split, int n_sparse_wg,
                                                             float* __restrict__ o_part, float* __restrict__ lse_part,
                                                             LocalArgs la, int n_split_loc, float* __restrict__ ws_o,
                                                             float* __restrict__ ws_lse) {
  __shared__ union {
    SparseSmem<G> s;
    LocalSmem<G> l;
  } S;
  const int id = blockIdx.x;
  if (id < n_sparse_wg) {
    const int c = id % n_split;
    const SparseGroup<G> grp = sparse_group<G>(a, B, id / n_split, &S.s);
    const int b = grp.b, n_ret = a.n_ret;
    sparse_split<BK, G>(a, c, grp, &S.s, [&](int i, int d, float o, float lse) {
      const size_t hr = (size_t)b * n_ret + i;
      o_part[(hr * n_split + c) * kHeadDim + d] = o;
      if (d == 0) lse_part[hr * n_split + c] = lse;
    });
  } else {
    const int j = id - n_sparse_wg;
    const int c = j % n_split_loc, gb = j / n_split_loc;
    const int g = gb % la.Hkv, b = gb / la.Hkv;
    const int n_loc = la.n_loc;
    local_split<G>(la, c, g, b, &S.l, [&](int i, int d, float o, float lse) {
      const size_t hr = (size_t)b * n_loc + i;
      ws_o[(hr * n_split_loc + c) * kHeadDim + d] = o;
      if (d == 0) ws_lse[hr * n_split_loc + c] = lse;
    });
  }
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
  if (!out) return RTP_EINVAL;
  LocalLayout L{};
  const rtp_status chk = local_args_check(q, k_cache, v_cache, seq_lens, loc_heads, B, Hq, Hkv, n_loc, max_ctx, window,
                                          sinks, workspace, ws_bytes, kv_slot, n_full, k_ring, v_ring, n_ring,
                                          local_layout, L);
  if (chk != RTP_OK) return chk;
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

namespace {

template <int BK>
void launch_step_attn(int G, int n_wg, hipStream_t s, const SparseArgs& a, int B, int n_split, int n_sparse_wg,
                      float* op, float* lp, const LocalArgs& la, int n_split_loc, float* wo, float* wl) {
#define RTP_STEP(GG)                                                                                      \
  hipLaunchKernelGGL((step_attn_kernel<BK, GG>), dim3(n_wg), dim3(kThreads), 0, s, a, B, n_split, n_sparse_wg, \
                     op, lp, la, n_split_loc, wo, wl)
  switch (G) {
    case 1: RTP_STEP(1); break;
    case 2: RTP_STEP(2); break;
    case 4: RTP_STEP(4); break;
    default: RTP_STEP(8); break;
  }
#undef RTP_STEP
}

}  // namespace

extern "C" rtp_status rtp_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                                      const int* ret_heads, const int* sel_idx, const int* sel_cnt,
                                      const unsigned char* sel_mask, const int* loc_heads, int B, int Hq, int Hkv,
                                      int n_ret, int n_loc, int max_ctx, int block, int split_tokens, int window,
                                      int sinks, float* o_part, float* lse_part, void* ws_local,
                                      size_t ws_local_bytes, const int* kv_slot, int n_full, const void* k_ring,
                                      const void* v_ring, int n_ring, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_ctx <= 0 || n_ret < 0 || n_loc < 0 || n_ret + n_loc > Hq)
    return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (!group_ok(Hq, Hkv)) return RTP_EUNSUPPORTED;
  if (B > 65535) return RTP_EUNSUPPORTED;
  if (n_ret == 0 && n_loc == 0) return RTP_OK;
  if (!q || !seq_lens) return RTP_EINVAL;
  if (n_ret > 0) {
    if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
    if (split_tokens <= 0 || split_tokens % block) return RTP_EINVAL;
    if (split_tokens / block > kMaxSplitBlocks) return RTP_EUNSUPPORTED;
    if (ceil_div(max_ctx, split_tokens) > 65535) return RTP_EUNSUPPORTED;
    if (!ret_heads || !o_part || !lse_part || (!sel_mask && (!sel_idx || !sel_cnt))) return RTP_EINVAL;
    if (kv_slot && (n_full < 1 || n_full > Hkv)) return RTP_EINVAL;
    if (!k_cache || !v_cache || (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)) return RTP_EINVAL;
  }
  LocalLayout L{};
  L.n_split = 1;
  if (n_loc > 0) {
    const rtp_status chk = local_args_check(q, k_cache, v_cache, seq_lens, loc_heads, B, Hq, Hkv, n_loc, max_ctx,
                                            window, sinks, ws_local, ws_local_bytes, kv_slot, n_full, k_ring, v_ring,
                                            n_ring, local_layout, L);
    if (chk != RTP_OK) return chk;
  }
  const int n_split = n_ret > 0 ? ceil_div(max_ctx, split_tokens) : 1;
  const long long n_sparse_wg = n_ret > 0 ? (long long)n_split * Hkv * B : 0;
  const long long n_local_wg = n_loc > 0 ? (long long)L.n_split * Hkv * B : 0;
  if (n_sparse_wg + n_local_wg > 0x7FFFFFFFll) return RTP_EUNSUPPORTED;
  const int nblk_max = n_ret > 0 ? ceil_div(max_ctx, block) : 1;
  const SparseArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), seq_lens, ret_heads, sel_idx, sel_cnt, sel_mask, kv_slot,
                     Hq, Hkv, n_ret, max_ctx, nblk_max, n_ret > 0 ? split_tokens / block : 1,
                     kv_slot ? n_full : Hkv};
  char* ws = static_cast<char*>(ws_local);
  const LocalArgs la{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), seq_lens, loc_heads, Hq, Hkv, n_loc, max_ctx, window, sinks,
                     n_loc > 0 ? L.split_tokens : 1, kv_slot, static_cast<const uint16_t*>(k_ring),
                     static_cast<const uint16_t*>(v_ring), kv_slot ? n_full : Hkv, kv_slot ? n_ring : 0};
  float* wl = n_loc > 0 ? reinterpret_cast<float*>(ws + L.off_lse) : nullptr;
  float* wo = n_loc > 0 ? reinterpret_cast<float*>(ws + L.off_o) : nullptr;
  const int n_wg = (int)(n_sparse_wg + n_local_wg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (block == 128 && n_ret > 0)
    launch_step_attn<128>(Hq / Hkv, n_wg, s, a, B, n_split, (int)n_sparse_wg, o_part, lse_part, la, L.n_split, wo,
                          wl);
  else
    launch_step_attn<64>(Hq / Hkv, n_wg, s, a, B, n_split, (int)n_sparse_wg, o_part, lse_part, la, L.n_split, wo,
                         wl);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" rtp_status rtp_decode_merge(const float* o_part, const float* lse_part, const int* ret_heads,
                                       const int* loc_heads, int B, int Hq, int Hkv, int n_ret, int n_loc,
                                       int max_ctx, int split_tokens, int window, int sinks, const void* ws_local,
                                       size_t ws_local_bytes, float* out, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_ctx <= 0 || n_ret < 0 || n_loc < 0 || n_ret + n_loc > Hq)
    return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (B > 65535) return RTP_EUNSUPPORTED;
  if (n_ret + n_loc == 0) return RTP_OK;
  if (!out) return RTP_EINVAL;
  int n_split = 1;
  if (n_ret > 0) {
    if (split_tokens <= 0 || !o_part || !lse_part || !ret_heads) return RTP_EINVAL;
    n_split = ceil_div(max_ctx, split_tokens);
  }
  LocalLayout L{};
  L.n_split = 1;
  if (n_loc > 0) {
    if (window < 0 || sinks < 0 || window + sinks < 1 || !loc_heads || !ws_local) return RTP_EINVAL;
    L = local_layout(B, Hkv, n_loc, window < max_ctx ? window : max_ctx);
    if (ws_local_bytes < L.total) return RTP_EINVAL;
  }
  const char* ws = static_cast<const char*>(ws_local);
  hipLaunchKernelGGL(merge_step_kernel, dim3(n_ret + n_loc, B), dim3(kMergeThreads), 0,
                     static_cast<hipStream_t>(stream), o_part, lse_part, ret_heads, n_ret, n_split,
                     n_loc > 0 ? reinterpret_cast<const float*>(ws + L.off_o) : nullptr,
                     n_loc > 0 ? reinterpret_cast<const float*>(ws + L.off_lse) : nullptr, loc_heads, n_loc,
                     L.n_split, Hq, out);
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
