// Kernel 1 of the decode path: low-rank index scoring and exact block top-p.
//
// Index score s_n = (W^Q_r q_pre)^T k_idx_n with pre-RoPE features (RTPurbo review,
// Method / Adaptive sparse attention equation); the active set is the block-wise
// top-p of the score distribution, found by a histogram threshold that the last
// workgroup computes, fused with scoring in one launch (review, Hardware-aware
// top-p decoding kernel; "Full Attention Strikes Back" architecture paragraph:
// Kernel 1 at D16, 256-bin histogram, atomic counters).
//
// gfx950 design
//   grid (chunk, retrieval head, sequence), 256 threads = 4 wave64.
//   Scoring: each wave streams whole KV blocks of the 32 B/token index-key cache with
//   16-byte loads; one load instruction covers 1 KB (32 tokens, two lanes per token).
//   q_idx and the scores are fp64 so that block masses carry < 1e-6 relative error;
//   exponentials are fp32 hardware exp2 on arguments already reduced in fp64, summed
//   in fp64.  Per block: lse_j = max + log(sum exp(s - max)).  Per chunk: M_c, Z_c
//   and e_j = exp(lse_j - M_c) go to the workspace.
//   Selection: the last workgroup per (b, r) (device-scope release/acquire around an
//   atomic arrival counter, needed across the 8 XCDs' separate L2s) forms
//   m_j = e_j exp(M_c - M) / Z, takes the order-preserving bits of m_j as the radix
//   key (ties broken by block id, which extends the key), and runs 256-bin LDS
//   histograms of (count, fixed-point mass) from the most significant digit down.
//   Each pass keeps the bin where the cumulative mass crosses p; once the crossing
//   bin holds <= 64 blocks one wave ranks them exactly.  Masses are summed as
//   fixed-point integers (2^-62 units), so every cumulative sum is exact and the
//   result is deterministic.  The selected ids are written in ascending order by a
//   ballot-based ordered compaction, and the arrival counter is reset to zero.

#include "rtp_common.hpp"

namespace rtp {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunkBlocks = 128;
constexpr int kMaxChunks = 1024;
constexpr int kMaxBlocks = 1 << 17;     // nblk limit (also bounds the tie-break key)
constexpr int kResolve = 64;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct K1Layout {
  int nblk_max, chunk_blocks, chunk_shift, n_chunk;
  size_t off_counters, off_stats, off_e, total;
};

// Chunk size: aim for >= 2048 workgroups over the whole batch, 8..128 blocks a chunk,
// at most kMaxChunks chunks per head.
K1Layout k1_layout(int B, int n_ret, int max_ctx, int block) {
  K1Layout L{};
  L.nblk_max = ceil_div(max_ctx, block);
  long long total_blocks = (long long)B * n_ret * L.nblk_max;
  int cb = kMaxChunkBlocks;
  while (cb > 8 && total_blocks / cb < 2048) cb >>= 1;
  while (ceil_div(L.nblk_max, cb) > kMaxChunks && cb < kMaxChunkBlocks) cb <<= 1;
  L.chunk_blocks = cb;
  L.chunk_shift = __builtin_ctz(cb);
  L.n_chunk = ceil_div(L.nblk_max, cb);
  const size_t heads = (size_t)B * n_ret;
  L.off_counters = 0;
  L.off_stats = align_up(heads * sizeof(int), 256);
  L.off_e = L.off_stats + align_up(heads * L.n_chunk * 2 * sizeof(double), 256);
  L.total = L.off_e + align_up(heads * (size_t)L.nblk_max * sizeof(double), 256);
  return L;
}

// Radix digits of the composite key (hi = bits of the clamped fp64 mass, whose top
// three bits are always 001; lo = 0xFFFFFF - block id).
__constant__ int kShift[11] = {53, 45, 37, 29, 21, 13, 5, 0, 16, 8, 0};
__constant__ int kWidth[11] = {8, 8, 8, 8, 8, 8, 8, 5, 8, 8, 8};

struct Elem {
  uint64_t hi;
  uint32_t lo;
  uint64_t fm;
};

__device__ __forceinline__ Elem make_elem(double e, double f, int j) {
  const double m = e * f;
  Elem x;
  x.hi = (uint64_t)__double_as_longlong(fmax(m, 0x1p-511));
  x.lo = 0xFFFFFFu - (uint32_t)j;
  x.fm = (uint64_t)(m * 0x1p62);
  return x;
}

__device__ __forceinline__ bool geq(uint64_t hi, uint32_t lo, uint64_t thi, uint32_t tlo) {
  return hi > thi || (hi == thi && lo >= tlo);
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  uint32_t a = __shfl_up((uint32_t)v, d), b = __shfl_up((uint32_t)(v >> 32), d);
  return ((uint64_t)b << 32) | a;
}

template <int BK>
__global__ __launch_bounds__(kThreads) void index_topp_kernel(
    const uint16_t* __restrict__ q_pre, const uint16_t* __restrict__ w_q,
    const uint16_t* __restrict__ k_idx, const int* __restrict__ seq_lens,
    const int* __restrict__ ret_heads, const float* __restrict__ top_p, int Hq, int n_ret,
    int max_ctx, int nblk_max, int chunk_blocks, int chunk_shift, int n_chunk_max, int* __restrict__ sel_idx,
    int* __restrict__ sel_cnt, int* __restrict__ counters, double2* __restrict__ stats,
    double* __restrict__ blk_e) {
  constexpr int NL = BK / 32;              // 1 KB loads per lane per block
  constexpr int U = BK == 64 ? 2 : 1;      // blocks in flight per wave
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int N = seq_lens[b];
  const int nblk = (N + BK - 1) / BK;
  const int nch = (nblk + chunk_blocks - 1) / chunk_blocks;
  if (c >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head = (size_t)b * n_ret + r;

  __shared__ double s_qidx[kIndexDim];
  __shared__ double s_lse[kMaxChunkBlocks];
  __shared__ double s_f[kMaxChunks];
  __shared__ uint32_t s_hcnt[256];
  __shared__ uint64_t s_hmass[256];
  __shared__ uint64_t s_chi[kResolve];
  __shared__ uint32_t s_clo[kResolve];
  __shared__ uint64_t s_cfm[kResolve];
  __shared__ uint64_t s_shi[kResolve];
  __shared__ uint32_t s_slo[kResolve];
  __shared__ uint64_t s_sfm[kResolve];
  __shared__ double s_red[kWaves];
  __shared__ int s_wcnt[kWaves];
  __shared__ int s_flag;
  __shared__ int s_bin, s_bcnt, s_ncand;
  __shared__ uint64_t s_cab, s_thi;
  __shared__ uint32_t s_tlo;

  // ---- q_idx = W^Q_r q_pre[b, hq] in fp64 (16 outputs x 16 partial dot products)
  {
    const int hq = ret_heads[r];
    const int i = tid >> 4, part = tid & 15;
    const uint4 wv = ld16(w_q + ((size_t)r * kIndexDim + i) * kHeadDim + part * 8);
    const uint4 qv = ld16(q_pre + ((size_t)b * Hq + hq) * kHeadDim + part * 8);
    double a = (double)bf_lo(wv.x) * (double)bf_lo(qv.x);
    a = fma((double)bf_hi(wv.x), (double)bf_hi(qv.x), a);
    a = fma((double)bf_lo(wv.y), (double)bf_lo(qv.y), a);
    a = fma((double)bf_hi(wv.y), (double)bf_hi(qv.y), a);
    a = fma((double)bf_lo(wv.z), (double)bf_lo(qv.z), a);
    a = fma((double)bf_hi(wv.z), (double)bf_hi(qv.z), a);
    a = fma((double)bf_lo(wv.w), (double)bf_lo(qv.w), a);
    a = fma((double)bf_hi(wv.w), (double)bf_hi(qv.w), a);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o);
    if (part == 0) s_qidx[i] = a;
  }
  __syncthreads();
  const int half = lane & 1;
  double qh[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) qh[k] = s_qidx[half * 8 + k];

  // ---- scoring: lse of every block of this chunk
  const uint16_t* kb = k_idx + head * (size_t)max_ctx * kIndexDim + half * 8;
  const int j0 = c * chunk_blocks;
  const int j1 = min(j0 + chunk_blocks, nblk);
  for (int jj = j0 + wave; jj < j1; jj += kWaves * U) {
    uint4 v[U][NL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jj + u * kWaves;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int tok = j * BK + 32 * t + (lane >> 1);
        v[u][t] = (j < j1 && tok < N) ? ld16(kb + (size_t)tok * kIndexDim) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jj + u * kWaves;
      if (j >= j1) break;
      double s[NL];
      double m = -INFINITY;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const uint4 x = v[u][t];
        double a = qh[0] * (double)bf_lo(x.x);
        a = fma(qh[1], (double)bf_hi(x.x), a);
        a = fma(qh[2], (double)bf_lo(x.y), a);
        a = fma(qh[3], (double)bf_hi(x.y), a);
        a = fma(qh[4], (double)bf_lo(x.z), a);
        a = fma(qh[5], (double)bf_hi(x.z), a);
        a = fma(qh[6], (double)bf_lo(x.w), a);
        a = fma(qh[7], (double)bf_hi(x.w), a);
        a += __shfl_xor(a, 1);  // commutative: both lanes of the pair hold the same score
        const int tok = j * BK + 32 * t + (lane >> 1);
        s[t] = tok < N ? a : -INFINITY;
        m = fmax(m, s[t]);
      }
      m = wave_max(m);
      double sum = 0.0;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const float x = (float)((s[t] - m) * kLog2e);
        const double e = (double)fast_exp2(x);
        sum += half ? 0.0 : e;
      }
      sum = wave_sum(sum);
      if (lane == 0) s_lse[j - j0] = m + log(sum);
    }
  }
  __syncthreads();

  // ---- chunk epilogue: M_c, Z_c, e_j = exp(lse_j - M_c)
  if (wave == 0) {
    const int nb = j1 - j0;
    const double l0 = lane < nb ? s_lse[lane] : -INFINITY;
    const double l1 = lane + 64 < nb ? s_lse[lane + 64] : -INFINITY;
    const double Mc = wave_max(fmax(l0, l1));
    const double e0 = lane < nb ? exp(l0 - Mc) : 0.0;
    const double e1 = lane + 64 < nb ? exp(l1 - Mc) : 0.0;
    double* eb = blk_e + head * nblk_max + j0;
    if (lane < nb) eb[lane] = e0;
    if (lane + 64 < nb) eb[lane + 64] = e1;
    const double Zc = wave_sum(e0 + e1);
    if (lane == 0) stats[head * n_chunk_max + c] = make_double2(Mc, Zc);
  }
  __syncthreads();

  // ---- arrival: the last workgroup of (b, r) selects
  if (tid == 0) {
    __threadfence();  // release this workgroup's e_j and chunk stats device-wide
    const int prev = atomicAdd(&counters[head], 1);
    s_flag = prev == nch - 1;
    if (s_flag) __threadfence();  // acquire every other workgroup's results
  }
  __syncthreads();
  if (!s_flag) return;

  // ---- M, Z and the per-chunk factors f_c = exp(M_c - M) / Z
  const double2* st = stats + head * n_chunk_max;
  double mloc = -INFINITY;
  for (int i = tid; i < nch; i += kThreads) mloc = fmax(mloc, st[i].x);
  mloc = wave_max(mloc);
  if (lane == 0) s_red[wave] = mloc;
  __syncthreads();
  double M = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmax(M, s_red[w]);
  __syncthreads();
  double zloc = 0.0;
  for (int i = tid; i < nch; i += kThreads) {
    const double2 v = st[i];
    const double f = exp(v.x - M);
    s_f[i] = f;
    zloc += v.y * f;
  }
  zloc = wave_sum(zloc);
  if (lane == 0) s_red[wave] = zloc;
  __syncthreads();
  double Z = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) Z += s_red[w];
  const double invZ = 1.0 / Z;
  for (int i = tid; i < nch; i += kThreads) s_f[i] *= invZ;
  __syncthreads();

  const double* eb = blk_e + head * nblk_max;
  auto elem = [&](int j) { return make_elem(eb[j], s_f[j >> chunk_shift], j); };

  // threshold T: block j is selected iff (hi_j, lo_j) >= (thi, tlo)
  uint64_t thi = 0;
  uint32_t tlo = 0;
  const float p = top_p[head];
  if (p < 1.0f && nblk > 1) {
    const uint64_t P = (uint64_t)ceil(ldexp((double)p, 62));
    uint64_t pfx_hi = 1, cab = 0;  // prefix so far; fixed mass strictly above the candidates
    uint32_t pfx_lo = 0;
    bool done = false;
    for (int k = 0; k < 11 && !done; ++k) {
      const int sh = kShift[k], wd = kWidth[k], nbins = 1 << wd;
      for (int i = tid; i < 256; i += kThreads) {
        s_hcnt[i] = 0;
        s_hmass[i] = 0;
      }
      __syncthreads();
      for (int j = tid; j < nblk; j += kThreads) {
        const Elem x = elem(j);
        bool cand;
        uint32_t d;
        if (k < 8) {
          cand = (x.hi >> (sh + wd)) == pfx_hi;
          d = (uint32_t)(x.hi >> sh) & (nbins - 1);
        } else {
          cand = x.hi == pfx_hi && (x.lo >> (sh + wd)) == pfx_lo;
          d = (x.lo >> sh) & (nbins - 1);
        }
        if (cand) {
          atomicAdd(&s_hcnt[d], 1u);
          atomicAdd((unsigned long long*)&s_hmass[d], (unsigned long long)x.fm);
        }
      }
      __syncthreads();
      if (wave == 0) {
        // bins in descending order: lane L owns bins nbins-1-4L .. nbins-4-4L
        uint64_t bm[4];
        uint32_t bc[4];
        uint64_t tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bin = nbins - 1 - 4 * lane - q;
          bm[q] = bin >= 0 ? s_hmass[bin] : 0;
          bc[q] = bin >= 0 ? s_hcnt[bin] : 0;
          tot += bm[q];
        }
        uint64_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint64_t y = shfl_up_u64(incl, o);
          if (lane >= o) incl += y;
        }
        uint64_t run = cab + (incl - tot);
        int hit = -1;
        uint64_t hit_above = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (hit < 0 && run + bm[q] >= P && bm[q] > 0) {
            hit = q;
            hit_above = run;
          }
          run += bm[q];
        }
        const uint64_t any = __ballot(hit >= 0);
        const int first = any ? __builtin_ctzll(any) : -1;
        if (lane == 0 && first < 0) s_bin = -1;
        if (lane == first) {
          s_bin = nbins - 1 - 4 * lane - hit;
          s_bcnt = (int)bc[hit];
          s_cab = hit_above;
        }
      }
      __syncthreads();
      const int bin = s_bin;
      if (bin < 0) {  // no prefix reaches p (only possible on the first pass): select all
        thi = 0;
        tlo = 0;
        done = true;
        break;
      }
      cab = s_cab;
      const int bcnt = s_bcnt;
      if (k < 8) {
        pfx_hi = (pfx_hi << wd) | (uint64_t)bin;
      } else {
        pfx_lo = (pfx_lo << wd) | (uint32_t)bin;
      }
      if (bcnt == 1 || k == 10) {
        if (k < 8) {
          thi = pfx_hi << sh;
          tlo = 0;
        } else {
          thi = pfx_hi;
          tlo = pfx_lo << sh;
        }
        done = true;
      } else if (bcnt <= kResolve) {
        // gather the candidates and rank them exactly in one wave
        if (tid == 0) s_ncand = 0;
        __syncthreads();
        for (int j = tid; j < nblk; j += kThreads) {
          const Elem x = elem(j);
          const bool cand = k < 8 ? (x.hi >> sh) == pfx_hi : (x.hi == pfx_hi && (x.lo >> sh) == pfx_lo);
          if (cand) {
            const int slot = atomicAdd(&s_ncand, 1);
            s_chi[slot] = x.hi;
            s_clo[slot] = x.lo;
            s_cfm[slot] = x.fm;
          }
        }
        __syncthreads();
        const int nc = s_ncand;
        if (wave == 0 && lane < nc) {
          const uint64_t mh = s_chi[lane];
          const uint32_t ml = s_clo[lane];
          int rank = 0;
          for (int i = 0; i < nc; ++i) {
            const uint64_t oh = s_chi[i];
            const uint32_t ol = s_clo[i];
            rank += (oh > mh || (oh == mh && ol > ml)) ? 1 : 0;
          }
          s_shi[rank] = mh;   // ranks are a permutation of 0..nc-1
          s_slo[rank] = ml;
          s_sfm[rank] = s_cfm[lane];
        }
        __syncthreads();
        if (wave == 0) {
          const uint64_t f = lane < nc ? s_sfm[lane] : 0;
          uint64_t incl = f;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const uint64_t y = shfl_up_u64(incl, o);
            if (lane >= o) incl += y;
          }
          const bool cross = lane < nc && cab + incl >= P;
          const uint64_t any = __ballot(cross);
          const int first = any ? __builtin_ctzll(any) : nc - 1;
          if (lane == first) {
            s_thi = s_shi[lane];
            s_tlo = s_slo[lane];
          }
        }
        __syncthreads();
        thi = s_thi;
        tlo = s_tlo;
        done = true;
      }
      __syncthreads();
    }
  }

  // ---- ordered compaction of the selected ids (ascending), one contiguous segment a wave
  int* out = sel_idx + head * nblk_max;
  const int seg = ((nblk + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int sb = wave * seg, se = min(nblk, sb + seg);
  int cnt = 0;
  for (int base = sb; base < se; base += 64) {
    const int j = base + lane;
    bool sel = false;
    if (j < se) {
      const Elem x = elem(j);
      sel = geq(x.hi, x.lo, thi, tlo);
    }
    cnt += __popcll(__ballot(sel));
  }
  if (lane == 0) s_wcnt[wave] = cnt;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += s_wcnt[w];
  for (int base = sb; base < se; base += 64) {
    const int j = base + lane;
    bool sel = false;
    if (j < se) {
      const Elem x = elem(j);
      sel = geq(x.hi, x.lo, thi, tlo);
    }
    const uint64_t mask = __ballot(sel);
    if (sel) out[off + __popcll(mask & lanemask_lt())] = j;
    off += __popcll(mask);
  }
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < kWaves; ++w) total += s_wcnt[w];
    sel_cnt[head] = total;
    atomicExch(&counters[head], 0);  // ready for the next call
  }
}

}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" size_t rtp_index_topp_workspace_size(int B, int n_ret, int max_ctx, int block) {
  if (B <= 0 || n_ret <= 0 || max_ctx <= 0 || (block != 64 && block != 128)) return 0;
  if (ceil_div(max_ctx, block) > kMaxBlocks) return 0;
  return k1_layout(B, n_ret, max_ctx, block).total;
}

extern "C" rtp_status rtp_index_topp(const void* q_pre, const void* w_q, const void* k_idx,
                                     const int* seq_lens, const int* ret_heads, const float* top_p,
                                     int B, int Hq, int n_ret, int max_ctx, int block, int* sel_idx,
                                     int* sel_cnt, void* workspace, size_t ws_bytes, void* stream) {
  if (B <= 0 || Hq <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
  if (ceil_div(max_ctx, block) > kMaxBlocks) return RTP_EUNSUPPORTED;
  if (n_ret == 0) return RTP_OK;
  if (!q_pre || !w_q || !k_idx || !seq_lens || !ret_heads || !top_p || !sel_idx || !sel_cnt ||
      !workspace)
    return RTP_EINVAL;
  if (((uintptr_t)q_pre | (uintptr_t)w_q | (uintptr_t)k_idx) & 15) return RTP_EINVAL;
  if ((uintptr_t)workspace & 255) return RTP_EINVAL;
  const K1Layout L = k1_layout(B, n_ret, max_ctx, block);
  if (ws_bytes < L.total) return RTP_EINVAL;
  char* ws = static_cast<char*>(workspace);
  int* counters = reinterpret_cast<int*>(ws + L.off_counters);
  double2* stats = reinterpret_cast<double2*>(ws + L.off_stats);
  double* blk_e = reinterpret_cast<double*>(ws + L.off_e);
  dim3 grid(L.n_chunk, n_ret, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qp = static_cast<const uint16_t*>(q_pre);
  const uint16_t* wq = static_cast<const uint16_t*>(w_q);
  const uint16_t* ki = static_cast<const uint16_t*>(k_idx);
  if (block == 64)
    hipLaunchKernelGGL(index_topp_kernel<64>, grid, dim3(kThreads), 0, s, qp, wq, ki, seq_lens,
                       ret_heads, top_p, Hq, n_ret, max_ctx, L.nblk_max, L.chunk_blocks, L.chunk_shift, L.n_chunk,
                       sel_idx, sel_cnt, counters, stats, blk_e);
  else
    hipLaunchKernelGGL(index_topp_kernel<128>, grid, dim3(kThreads), 0, s, qp, wq, ki, seq_lens,
                       ret_heads, top_p, Hq, n_ret, max_ctx, L.nblk_max, L.chunk_blocks, L.chunk_shift, L.n_chunk,
                       sel_idx, sel_cnt, counters, stats, blk_e);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}
