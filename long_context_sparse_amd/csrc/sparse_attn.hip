// Kernel 2 of the decode path and the local heads' kernel.
//
// Kernel 2: exact softmax(q K^T / sqrt(128)) V over only the blocks the index kernel
// selected, split along the context ("Full Attention Strikes Back", method item 2 and
// architecture paragraph: Kernel 2 at D128 with a cross-split reduce).  Workgroup =
// (split, KV group, sequence); it builds the union of its retrieval heads' selected
// blocks inside the split (binary search into each ascending list, LDS head-mask per
// block, ordered compaction), so a block picked by several heads of the group is read
// from HBM once, then streams the union's 16-token sub-tiles through the shared
// attention core and writes per-head (o, lse) partials.
//
// Local heads: the same core over attention sinks + the sliding window (RTPurbo
// review, Adaptive sparse attention: local heads keep only window + sinks).
// Workgroup = (split, KV group, sequence); split 0 holds the sinks, splits 1.. hold
// consecutive window chunks.  Each workgroup writes per-head (o, lse) partials to the
// workspace, and a merge kernel (one workgroup per output row, the same kernel as the
// cross-split reduce) combines them with the log-sum-exp rule.

#include "rtp_attn.hpp"

namespace rtp {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSplitBlocks = 2048;

// Contiguous range [beg, end) of an ascending head list that falls in KV group g,
// found by one wave with 64 parallel loads per round (every lane gets the result).
__device__ __forceinline__ void group_range(const int* __restrict__ heads, int n, int g, int G,
                                            int& beg, int& end) {
  const int lane = threadIdx.x & 63;
  beg = 0;
  end = 0;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const int h = i < n ? heads[i] : 0x7fffffff;
    beg += __popcll(__ballot(h < g * G));
    end += __popcll(__ballot(h < (g + 1) * G));
  }
}

// First index of the ascending list a[0, n) whose value is >= key (n if none), found by
// one wave: each round probes 64 evenly spaced entries of the remaining range, so a
// list of 16K entries takes three rounds of parallel loads.
__device__ __forceinline__ int lower_bound_wave(const int* __restrict__ a, int n, int key) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;  // the answer lies in [lo, hi]
  while (lo < hi) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const int k = __popcll(__ballot(idx < hi && a[idx] < key));  // probes below key: a prefix
    if (k == 0) break;
    if (step == 1) {
      lo += k;
      break;
    }
    hi = min(hi, lo + k * step);
    lo += (k - 1) * step + 1;
  }
  return lo;
}

template <int BK, int G>
__global__ __launch_bounds__(kThreads) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int* __restrict__ seq_lens, const int* __restrict__ ret_heads,
    const int* __restrict__ sel_idx, const int* __restrict__ sel_cnt, int Hq, int Hkv, int n_ret,
    int max_ctx, int nblk_max, int split_blocks, int n_split, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  constexpr int ST = BK / 16;  // sub-tiles per block
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the first 64 selected counts go out with the head list (one memory round trip)
  const int cnt_l = lane < n_ret ? sel_cnt[(size_t)b * n_ret + lane] : 0;
  int rbeg, rend;
  group_range(ret_heads, n_ret, g, G, rbeg, rend);
  const int nh = rend - rbeg;
  if (nh == 0) return;
  const int N = seq_lens[b];
  const int nblk = (N + BK - 1) / BK;
  const int jlo = c * split_blocks, jhi = min(jlo + split_blocks, nblk);

  __shared__ uint32_t s_hm[kMaxSplitBlocks / 4];
  __shared__ uint32_t s_list[kMaxSplitBlocks];
  __shared__ int s_wcnt[kWaves];
  __shared__ float s_m[kWaves * G], s_l[kWaves * G];
  __shared__ float s_acc[kWaves * G * kHeadDim];

  int nL = 0;
  if (jlo < jhi) {
    const int nb = jhi - jlo;
    for (int i = tid; i < (nb + 3) / 4; i += kThreads) s_hm[i] = 0;
    __syncthreads();
    // mark each head's selected blocks in [jlo, jhi): one wave per head.  A list of at
    // most 64 entries is read in one round; a longer one is searched for its range.
    for (int h = wave; h < nh; h += kWaves) {
      const int hh = rbeg + h;
      const size_t hr = (size_t)b * n_ret + hh;
      const int cnt = hh < 64 ? __shfl(cnt_l, hh) : sel_cnt[hr];
      const int* sl = sel_idx + hr * nblk_max;
      const uint32_t bit = 1u << h;
      if (cnt <= 64) {
        const int v = lane < cnt ? sl[lane] : -1;
        if (v >= jlo && v < jhi) atomicOr(&s_hm[(v - jlo) >> 2], bit << (((v - jlo) & 3) * 8));
      } else {
        const int a = lower_bound_wave(sl, cnt, jlo);
        const int e = lower_bound_wave(sl, cnt, jhi);
        for (int i = a + lane; i < e; i += 64) {
          const int off = sl[i] - jlo;
          atomicOr(&s_hm[off >> 2], bit << ((off & 3) * 8));
        }
      }
    }
    __syncthreads();
    // ordered compaction of the blocks some head selected: entry = (offset << 8) | mask
    const int seg = ((nb + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int sb = wave * seg, se = min(nb, sb + seg);
    int cnt = 0;
    for (int base = sb; base < se; base += 64) {
      const int off = base + lane;
      const uint32_t mk = off < se ? (s_hm[off >> 2] >> ((off & 3) * 8)) & 0xffu : 0u;
      cnt += __popcll(__ballot(mk != 0));
    }
    if (lane == 0) s_wcnt[wave] = cnt;
    __syncthreads();
    int pos = 0;
    for (int w = 0; w < wave; ++w) pos += s_wcnt[w];
    for (int base = sb; base < se; base += 64) {
      const int off = base + lane;
      const uint32_t mk = off < se ? (s_hm[off >> 2] >> ((off & 3) * 8)) & 0xffu : 0u;
      const uint64_t bal = __ballot(mk != 0);
      if (mk) s_list[pos + __popcll(bal & lanemask_lt())] = ((uint32_t)off << 8) | mk;
      pos += __popcll(bal);
    }
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) nL += s_wcnt[w];
  }

  AttnState<G> st;
  attn_init(st);
  uint4 qk[G];
  const int c16 = lane & 15;
#pragma unroll
  for (int h = 0; h < G; ++h)
    qk[h] = h < nh ? ld16(q + ((size_t)b * Hq + ret_heads[rbeg + h]) * kHeadDim + c16 * 8)
                   : make_uint4(0, 0, 0, 0);
  const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)max_ctx * kHeadDim;
  const float scale = (float)(kLog2e / 11.313708498984761);  // log2(e) / sqrt(128)
  auto item = [&](int i, int& row0, uint32_t& hm) {
    const uint32_t ent = s_list[i / ST];
    row0 = (jlo + (int)(ent >> 8)) * BK + 16 * (i % ST);
    hm = row0 < N ? (ent & 0xffu) : 0u;
  };
  attn_stream<G, kWaves>(st, kc + kvoff, vc + kvoff, nL * ST, N, item, qk, scale, wave, lane);
  attn_publish_wave<G, kWaves>(st, s_m, s_l, s_acc, wave, lane);
  __syncthreads();
  for (int idx = tid; idx < nh * kHeadDim; idx += kThreads) {
    const int h = idx >> 7, d = idx & (kHeadDim - 1);
    float o, lse;
    attn_merge<G, kWaves>(s_m, s_l, s_acc, h, d, o, lse);
    const size_t hr = (size_t)b * n_ret + rbeg + h;
    o_part[(hr * n_split + c) * kHeadDim + d] = o;
    if (d == 0) lse_part[hr * n_split + c] = lse;
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void local_window_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int* __restrict__ seq_lens, const int* __restrict__ loc_heads, int Hq, int Hkv, int n_loc,
    int max_ctx, int window, int sinks, int split_tokens, int n_split, float* __restrict__ ws_o,
    float* __restrict__ ws_lse) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int ibeg, iend;
  group_range(loc_heads, n_loc, g, G, ibeg, iend);
  const int nh = iend - ibeg;
  if (nh == 0) return;
  const int N = seq_lens[b];
  const int s_end = min(sinks, N);
  const int w0 = max(s_end, N - window);
  int t0, t1;
  if (c == 0) {
    t0 = 0;
    t1 = s_end;
  } else {
    t0 = w0 + (c - 1) * split_tokens;
    t1 = min(N, t0 + split_tokens);
  }
  const int nitems = t1 > t0 ? (t1 - t0 + 15) / 16 : 0;

  __shared__ float s_m[kWaves * G], s_l[kWaves * G];
  __shared__ float s_acc[kWaves * G * kHeadDim];

  AttnState<G> st;
  attn_init(st);
  uint4 qk[G];
  const int c16 = lane & 15;
#pragma unroll
  for (int h = 0; h < G; ++h)
    qk[h] = h < nh ? ld16(q + ((size_t)b * Hq + loc_heads[ibeg + h]) * kHeadDim + c16 * 8)
                   : make_uint4(0, 0, 0, 0);
  const size_t kvoff = ((size_t)b * Hkv + g) * (size_t)max_ctx * kHeadDim;
  const float scale = (float)(kLog2e / 11.313708498984761);
  const uint32_t allh = (1u << nh) - 1u;
  auto item = [&](int i, int& row0, uint32_t& hm) {
    row0 = t0 + 16 * i;
    hm = allh;
  };
  attn_stream<G, kWaves>(st, kc + kvoff, vc + kvoff, nitems, t1, item, qk, scale, wave, lane);
  attn_publish_wave<G, kWaves>(st, s_m, s_l, s_acc, wave, lane);
  __syncthreads();
  for (int idx = tid; idx < nh * kHeadDim; idx += kThreads) {
    const int h = idx >> 7, d = idx & (kHeadDim - 1);
    float o, lse;
    attn_merge<G, kWaves>(s_m, s_l, s_acc, h, d, o, lse);
    const size_t hr = (size_t)b * n_loc + ibeg + h;
    ws_o[(hr * n_split + c) * kHeadDim + d] = o;
    if (d == 0) ws_lse[hr * n_split + c] = lse;
  }
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

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Window split: >= ~1024 workgroups over the batch, 64..4096 tokens a split.
LocalLayout local_layout(int B, int Hkv, int n_loc, int window) {
  LocalLayout L{};
  const long long groups = (long long)B * Hkv;
  int st = 4096;
  while (st > 64 && groups * ceil_div(max(window, 1), st) < 1024) st >>= 1;
  L.split_tokens = st;
  L.n_split = 1 + ceil_div(window, st);
  L.off_lse = 0;
  L.off_o = align256((size_t)B * n_loc * L.n_split * sizeof(float));
  L.total = L.off_o + align256((size_t)B * n_loc * L.n_split * kHeadDim * sizeof(float));
  return L;
}

inline bool group_ok(int Hq, int Hkv) {
  if (Hkv <= 0 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

template <int BK>
void launch_sparse(int G, dim3 grid, hipStream_t s, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const int* sl, const int* rh, const int* si, const int* sc,
                   int Hq, int Hkv, int n_ret, int max_ctx, int nblk_max, int sb, int n_split,
                   float* op, float* lp) {
#define RTP_SPARSE(GG)                                                                        \
  hipLaunchKernelGGL((sparse_attn_kernel<BK, GG>), grid, dim3(kThreads), 0, s, q, k, v, sl, rh, \
                     si, sc, Hq, Hkv, n_ret, max_ctx, nblk_max, sb, n_split, op, lp)
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
                                            const int* sel_idx, const int* sel_cnt, int B, int Hq,
                                            int Hkv, int n_ret, int max_ctx, int block,
                                            int split_tokens, float* o_part, float* lse_part,
                                            void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (!group_ok(Hq, Hkv)) return RTP_EUNSUPPORTED;
  if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
  if (split_tokens <= 0 || split_tokens % block) return RTP_EINVAL;
  if (split_tokens / block > kMaxSplitBlocks) return RTP_EUNSUPPORTED;
  if (n_ret == 0) return RTP_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !ret_heads || !sel_idx || !sel_cnt || !o_part ||
      !lse_part)
    return RTP_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return RTP_EINVAL;
  const int nblk_max = ceil_div(max_ctx, block);
  const int sb = split_tokens / block;
  const int n_split = ceil_div(max_ctx, split_tokens);
  if (n_split > 65535) return RTP_EUNSUPPORTED;
  dim3 grid(n_split, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vv = static_cast<const uint16_t*>(v_cache);
  const int G = Hq / Hkv;
  if (block == 64)
    launch_sparse<64>(G, grid, s, qq, kk, vv, seq_lens, ret_heads, sel_idx, sel_cnt, Hq, Hkv, n_ret,
                      max_ctx, nblk_max, sb, n_split, o_part, lse_part);
  else
    launch_sparse<128>(G, grid, s, qq, kk, vv, seq_lens, ret_heads, sel_idx, sel_cnt, Hq, Hkv,
                       n_ret, max_ctx, nblk_max, sb, n_split, o_part, lse_part);
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
                                            void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_loc < 0 || n_loc > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv || window < 0 || sinks < 0 || window + sinks < 1) return RTP_EINVAL;
  if (!group_ok(Hq, Hkv)) return RTP_EUNSUPPORTED;
  if (n_loc == 0) return RTP_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !loc_heads || !out || !workspace) return RTP_EINVAL;
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
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vv = static_cast<const uint16_t*>(v_cache);
#define RTP_LOCAL(GG)                                                                         \
  hipLaunchKernelGGL(local_window_kernel<GG>, grid, dim3(kThreads), 0, s, qq, kk, vv, seq_lens, \
                     loc_heads, Hq, Hkv, n_loc, max_ctx, window, sinks, L.split_tokens,          \
                     L.n_split, ws_o, ws_lse)
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
    default: return "RTP_UNKNOWN";
  }
}

extern "C" const char* rtp_version(void) { return "rtp 1.0 gfx950"; }
