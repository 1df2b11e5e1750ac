// Kernel 1 of the decode path: low-rank index scoring and exact block top-p.
//
// Index score s_n = (W^Q_r q_pre)^T k_idx_n with pre-RoPE features (RTPurbo review,
// Method / Adaptive sparse attention equation); the active set is the block-wise
// top-p of the score distribution, found by a histogram threshold that the last
// workgroup computes, fused with scoring in one launch (review, Hardware-aware
// top-p decoding kernel; "Full Attention Strikes Back" architecture paragraph:
// Kernel 1 at D16, histogram threshold, atomic counters).
//
// gfx950 design
//   grid (chunk, retrieval head, sequence), 512 threads = 8 wave64.
//   Scoring: each wave streams whole KV blocks of the 32 B/token index-key cache with
//   16-byte loads; one load instruction covers 1 KB (32 tokens, two lanes per token).
//   q_idx and the scores are fp64 so that block masses carry < 1e-6 relative error;
//   exponentials are fp32 hardware exp2 on arguments already reduced in fp64, summed
//   in fp64; wave reductions run on DPP lane moves.  Per block: max_j and
//   sum_j = sum exp(s - max_j); per chunk M_c = max_j max_j, and the chunk publishes
//   e_j = sum_j exp(max_j - M_c) (fp32) and M_c (tagged fp64) to the workspace.
//   Publication without fences: every published 64-bit word carries the call's tag
//   (1..4095, advanced by every call) in its low 12 bits (the low mantissa bits of an
//   fp64, or beside an fp32), words are written and read with relaxed device-scope
//   atomics, and the reader waits for the current tag.
//   Every workgroup then bumps an arrival counter; the last one of each (b, r) does
//   the selection.  So no device-scope fence (an L2 write-back on every workgroup of
//   every XCD) is needed, and a word from the previous call is never taken as current.
//   Selection (last workgroup): M = max_c M_c, Z = sum_c Z_c exp(M_c - M) and every
//   block's mass m_j = e_j exp(M_c - M) / Z in fp32 into LDS, then the greedy
//   threshold exactly: a key = (fp32
//   mass bits, inverted block id) orders blocks by mass with ties by ascending id;
//   masses are summed as fixed-point integers (2^-62 units) so every cumulative sum
//   is exact and order-independent.  While more than 64 candidates of unequal mass
//   remain, a 256-bin LDS histogram of (count, mass) over (bits - lo) >> shift (bins
//   about log-uniform in mass) finds the bin where the cumulative mass crosses p, whose
//   bit range becomes the new candidate range (>= 128x narrower); the last <= 64
//   candidates are ranked exactly by one wave, and a run of equal masses is resolved by
//   count in ascending block order.  The selected ids are written in ascending order by
//   a ballot-based ordered compaction; the arrival counter is reset and the tag
//   advanced.

#include "rtp_common.hpp"

namespace rtp {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunkBlocks = 128;
constexpr int kMaxChunks = 1024;  // two per thread in the selection
constexpr int kMaxRows = 32;                  // blocks per thread in the selection
constexpr int kMaxBlocks = kMaxRows * kThreads;
constexpr int kBins = 256;                    // histogram bins per refinement level
constexpr int kFinal = kWave;                 // candidates ranked directly (one per lane)
constexpr int kSpinBudget = 1 << 12;          // re-reads a thread may spend waiting for a tag
constexpr uint64_t kTagBits = 0xFFFull;
static_assert(kMaxChunks == 2 * kThreads, "the selection reads two chunk records per thread");

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct K1Layout {
  int nblk_max, chunk_blocks, n_chunk, rows;
  size_t off_counters, off_tag, off_cmax, off_e, total;
};

// Chunk size: aim for >= 512 workgroups over the whole batch, 8..128 blocks a chunk,
// at most kMaxChunks chunks per head.  rows = blocks per thread in the selection.
K1Layout k1_layout(int B, int n_ret, int max_ctx, int block) {
  K1Layout L{};
  L.nblk_max = ceil_div(max_ctx, block);
  long long total_blocks = (long long)B * n_ret * L.nblk_max;
  int cb = kMaxChunkBlocks;
  while (cb > 8 && total_blocks / cb < 512) cb >>= 1;
  while (ceil_div(L.nblk_max, cb) > kMaxChunks && cb < kMaxChunkBlocks) cb <<= 1;
  L.chunk_blocks = cb;
  L.n_chunk = ceil_div(L.nblk_max, cb);
  L.rows = ceil_div(L.nblk_max, kThreads);
  const size_t heads = (size_t)B * n_ret;
  L.off_counters = 0;
  L.off_tag = align_up(heads * sizeof(int), 256);
  L.off_cmax = L.off_tag + align_up(heads * sizeof(uint32_t), 256);
  L.off_e = L.off_cmax + align_up(heads * L.n_chunk * 2 * sizeof(uint64_t), 256);
  L.total = L.off_e + align_up(heads * (size_t)L.nblk_max * sizeof(uint64_t), 256);
  return L;
}

// ------------------------------------------------------------------ published words
// fp64 values passed from the scoring workgroups to the selecting one: the low 12
// mantissa bits hold the call's tag (relative precision 2^-40 remains).
__device__ __forceinline__ uint64_t tagged(double x, uint32_t tag) {
  return ((uint64_t)__double_as_longlong(x) & ~kTagBits) | tag;
}
__device__ __forceinline__ double untag(uint64_t w) { return __longlong_as_double((long long)(w & ~kTagBits)); }
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Re-read a published word until it carries `tag` (bounded by the thread's budget).
__device__ __forceinline__ uint64_t settle(const uint64_t* p, uint64_t w, uint32_t tag, int& budget) {
  while ((uint32_t)(w & kTagBits) != tag && budget > 0) {
    --budget;
    __builtin_amdgcn_s_sleep(1);
    w = ld_dev(p);
  }
  return w;
}

// ------------------------------------------------------------------ selection helpers
// Composite selection key of block j with fp32 mass m >= 0: the mass bits (order-
// preserving for non-negative floats) above the inverted block id, so that keys are
// distinct and descending key order is descending mass with ties by ascending id.
__device__ __forceinline__ uint64_t key_of(float m, int j) {
  return ((uint64_t)__float_as_uint(m) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
// Mass in fixed point, 2^-62 units: integer sums are exact and order-independent.
__device__ __forceinline__ uint64_t fixed_mass(float m) { return (uint64_t)((double)m * 0x1p62); }

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t b = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)b << 32) | a;
}

struct TailSmem {
  uint64_t bmass[kBins];          // per bin: fixed-point mass
  uint32_t bcnt[kBins];           // per bin: candidate count
  int rowtab[kMaxRows * kWaves];  // per (row, wave) counts, then exclusive prefixes
  uint64_t u64[kWaves];
  double f64[kWaves], f64b[kWaves];
  uint32_t u32a[kWaves], u32b[kWaves];
  uint64_t ckey[kFinal], cfm[kFinal];  // final candidates (any order)
  uint64_t cab, thr;
  uint32_t lo, hi;
  int cnt, nfin, total;
};

template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o));
  return v;
}

// Reduction over the workgroup; every thread gets the result.
template <class T, class Op>
__device__ __forceinline__ T block_reduce(T v, T* red, Op op) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_reduce(v, op);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T t = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = op(t, red[w]);
  __syncthreads();
  return t;
}

struct SumOp {
  template <class T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct MinOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct MaxOp {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

// Exclusive prefix sum over the workgroup in thread order; `total` gets the sum.
template <class T>
__device__ __forceinline__ T block_excl_scan(T v, T* red, T& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  T base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    base += w < wave ? red[w] : T(0);
    total += red[w];
  }
  __syncthreads();
  return base + incl - v;
}

// Selection rows: block j = row * kThreads + thread, row < rows, masses in LDS (< 0 for
// no block).  Every pass reads a thread's masses kRowBatch rows at a time so the LDS
// latencies overlap.
constexpr int kRowBatch = 8;

template <class F>
__device__ __forceinline__ void for_rows(const float* __restrict__ sm_m, int rows, F f) {
  const int tid = threadIdx.x;
  for (int i0 = 0; i0 < rows; i0 += kRowBatch) {
    float mm[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) mm[u] = i0 + u < rows ? sm_m[(i0 + u) * kThreads + tid] : -1.0f;
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u)
      if (i0 + u < rows) f(i0 + u, mm[u]);
  }
}

// For a predicate on (row, mass), fills rowtab with the exclusive prefix, in ascending
// block order, of the satisfying blocks per (row, wave) and returns their total; the
// ordinal of a satisfying block is then rowtab[row * kWaves + wave] + (satisfying
// lanes below it in its wave).  One wave scans the table.
template <class Pred>
__device__ __forceinline__ int rows_prefix(const float* __restrict__ sm_m, int rows, Pred pred,
                                           TailSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for_rows(sm_m, rows, [&](int i, float m) {
    const uint64_t bal = __ballot(pred(i, m));
    if (lane == 0) sm.rowtab[i * kWaves + wave] = __popcll(bal);
  });
  __syncthreads();
  if (wave == 0) {
    constexpr int R = (kMaxRows * kWaves + 63) / 64;  // table entries a lane
    const int n = rows * kWaves;
    int v[R], tot = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int idx = lane * R + k;
      v[k] = idx < n ? sm.rowtab[idx] : 0;
      tot += v[k];
    }
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int run = incl - tot;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int idx = lane * R + k;
      if (idx < n) sm.rowtab[idx] = run;
      run += v[k];
    }
    if (lane == 63) sm.total = incl;
  }
  __syncthreads();
  return sm.total;
}

__device__ __forceinline__ int ordinal(bool flag, int i, const TailSmem& sm) {
  const int wave = threadIdx.x >> 6;
  return sm.rowtab[i * kWaves + wave] + __popcll(__ballot(flag) & lanemask_lt());
}

__device__ __forceinline__ uint64_t key_at(int i, float m) {
  return key_of(m, i * kThreads + (int)threadIdx.x);
}

// Exact greedy top-p threshold over the masses in LDS.  Returns the key of the last
// admitted block: the selected set is every block whose key is >= it.  Preconditions:
// the total fixed-point mass reaches P; [lo, hi] spans the mass bits of all blocks;
// the bins and the final-candidate count are zero.
//
// Candidates are the blocks whose mass bits lie in [lo, hi], with fixed mass `cab`
// strictly above them, and cab < P <= cab + mass(candidates) holds throughout.  A
// level puts every candidate into one of kBins bins by (bits - lo) >> shift, a
// monotone map, so bins are contiguous ranges of mass (about log-uniform, since fp32
// bits grow with log2 of the value); one wave scans the bins from the top, finds the
// bin where cab + cumulative mass crosses P, takes its bit range as the new candidate
// range (at least kBins/2 times narrower) and clears the bins.  It ends when <= kFinal
// candidates remain (ranked exactly by one wave), or when the range is a single mass
// value: the threshold is then the k-th candidate in ascending block order,
// k = ceil((P - cab) / mass).
__device__ uint64_t select_threshold(const float* __restrict__ sm_m, int rows, int nblk, uint64_t P,
                                     uint32_t lo, uint32_t hi, TailSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t cab = 0;
  int cnt = nblk;
  auto cand = [&](float m) {
    const uint32_t bits = __float_as_uint(m);
    return m >= 0.f && bits >= lo && bits <= hi;
  };
  while (cnt > kFinal && lo < hi) {
    const uint32_t span = hi - lo;
    const int shift = max(0, 32 - (int)__clz(span) - 8);  // (span >> shift) < kBins
    for_rows(sm_m, rows, [&](int i, float m) {
      if (cand(m)) {
        const int bin = (int)((__float_as_uint(m) - lo) >> shift);
        atomicAdd((unsigned long long*)&sm.bmass[bin], (unsigned long long)fixed_mass(m));
        atomicAdd(&sm.bcnt[bin], 1u);
      }
    });
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins kBins-1-4l .. kBins-4-4l (descending mass)
      uint64_t bm[4], run;
      uint32_t bc[4];
      uint64_t tot = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int bin = kBins - 1 - 4 * lane - k;
        bm[k] = sm.bmass[bin];
        bc[k] = sm.bcnt[bin];
        tot += bm[k];
        sm.bmass[bin] = 0;  // cleared for the next level
        sm.bcnt[bin] = 0;
      }
      uint64_t incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      run = cab + incl - tot;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (bm[k] > 0 && run < P && run + bm[k] >= P) {
          const uint32_t bin = kBins - 1 - 4 * lane - k;
          const uint32_t blo = lo + (bin << shift);
          sm.cab = run;
          sm.cnt = (int)bc[k];
          sm.lo = blo;
          sm.hi = min(hi, blo + ((1u << shift) - 1u));
        }
        run += bm[k];
      }
    }
    __syncthreads();
    cab = uni64(sm.cab);
    cnt = __builtin_amdgcn_readfirstlane(sm.cnt);
    lo = __builtin_amdgcn_readfirstlane(sm.lo);
    hi = __builtin_amdgcn_readfirstlane(sm.hi);
  }
  if (tid == 0) sm.thr = 0;
  if (cnt > kFinal) {
    // every candidate has mass bits lo: admit them in ascending block order
    auto tie = [&](int i, float m) { return m >= 0.f && __float_as_uint(m) == lo; };
    rows_prefix(sm_m, rows, tie, sm);
    const uint64_t f = fixed_mass(__uint_as_float(lo));
    if (f == 0) return 0;  // cannot happen while the invariant holds
    const uint64_t k = (P - cab + f - 1) / f;  // >= 1, <= cnt
    for_rows(sm_m, rows, [&](int i, float m) {
      const bool c = tie(i, m);
      const int ord = ordinal(c, i, sm);
      if (c && (uint64_t)ord + 1 == k) sm.thr = key_at(i, m);
    });
    __syncthreads();
    return uni64(sm.thr);
  }
  // the last <= kFinal candidates: gathered in any order, ranked by key in one wave
  // (keys are distinct, so the order is unique), then scanned from the top
  for_rows(sm_m, rows, [&](int i, float m) {
    if (cand(m)) {
      const int slot = atomicAdd(&sm.nfin, 1);
      sm.ckey[slot] = key_at(i, m);
      sm.cfm[slot] = fixed_mass(m);
    }
  });
  __syncthreads();
  if (wave == 0) {
    const int nf = sm.nfin;
    const uint64_t my = lane < nf ? sm.ckey[lane] : 0ull;
    const uint64_t f = lane < nf ? sm.cfm[lane] : 0ull;
    uint64_t above = 0;  // mass of the candidates with a larger key
    for (int i = 0; i < nf; ++i) above += sm.ckey[i] > my ? sm.cfm[i] : 0ull;
    if (lane < nf && cab + above < P && cab + above + f >= P) sm.thr = my;
    if (lane == 0) sm.nfin = 0;
  }
  __syncthreads();
  return uni64(sm.thr);
}

template <int BK>
__global__ __launch_bounds__(kThreads) void index_topp_kernel(
    const uint16_t* __restrict__ q_pre, const uint16_t* __restrict__ w_q,
    const uint16_t* __restrict__ k_idx, const int* __restrict__ seq_lens,
    const int* __restrict__ ret_heads, const float* __restrict__ top_p, int Hq, int n_ret,
    int max_ctx, int nblk_max, int chunk_blocks, int n_chunk_max, int* __restrict__ sel_idx,
    int* __restrict__ sel_cnt, int* __restrict__ counters, uint32_t* __restrict__ tags,
    uint64_t* __restrict__ cmax, uint64_t* __restrict__ blk_e) {
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
  __shared__ double s_mx[kMaxChunkBlocks], s_sum[kMaxChunkBlocks];  // scoring: per-block max, sum
  __shared__ double s_f[kMaxChunks];  // selection: per-chunk factor exp(M_c - M) / Z
  __shared__ TailSmem sm;
  __shared__ int s_flag;
  __shared__ uint32_t s_tag;
  extern __shared__ float s_mass[];  // selection: one fp32 mass per block (rows * kThreads)

  // ---- scoring: max and sum of every block of this chunk into LDS.  Wave w takes blocks
  // j0 + w + kWaves * (U * k + u); the next U blocks' loads are in flight while the
  // current U blocks are reduced.
  const int half = lane & 1;
  const uint16_t* kb = k_idx + head * (size_t)max_ctx * kIndexDim + half * 8;
  const int j0 = c * chunk_blocks;
  const int j1 = min(j0 + chunk_blocks, nblk);
  auto load = [&](uint4 (&v)[U][NL], int jj) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jj + u * kWaves;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int tok = j * BK + 32 * t + (lane >> 1);
        v[u][t] = (j < j1 && tok < N) ? ld16(kb + (size_t)tok * kIndexDim) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // the first blocks' loads go out before q_idx is formed
  int jj = j0 + wave;
  uint4 cur[U][NL];
  if (jj < j1) load(cur, jj);

  // ---- this call's tag; q_idx = W^Q_r q_pre[b, hq] in fp64 (16 outputs x 16 partial dots)
  if (tid == 0) {
    const uint32_t t = __hip_atomic_load(&tags[head], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_tag = t == 0 ? 1u : t;
  }
  if (tid < 256) {
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
  const uint32_t tag = s_tag;
  double qh[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) qh[k] = s_qidx[half * 8 + k];

  if (jj < j1) {
    while (true) {
      const int jn = jj + kWaves * U;
      uint4 nxt[U][NL];
      if (jn < j1) load(nxt, jn);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jj + u * kWaves;
        if (j >= j1) break;
        // scores in fp64, two 4-term chains per lane, then the pair sum (both lanes of
        // the pair then hold the token's score)
        double sc[NL];
        float mxf = -INFINITY;
#pragma unroll
        for (int t = 0; t < NL; ++t) {
          const uint4 x = cur[u][t];
          double a0 = qh[0] * (double)bf_lo(x.x);
          double a1 = qh[1] * (double)bf_hi(x.x);
          a0 = fma(qh[2], (double)bf_lo(x.y), a0);
          a1 = fma(qh[3], (double)bf_hi(x.y), a1);
          a0 = fma(qh[4], (double)bf_lo(x.z), a0);
          a1 = fma(qh[5], (double)bf_hi(x.z), a1);
          a0 = fma(qh[6], (double)bf_lo(x.w), a0);
          a1 = fma(qh[7], (double)bf_hi(x.w), a1);
          double a = a0 + a1;
          a += dpp_f64<kDppXor1>(a);  // commutative: both lanes of the pair get the same value
          const int tok = j * BK + 32 * t + (lane >> 1);
          sc[t] = tok < N ? a : -INFINITY;
          mxf = fmaxf(mxf, (float)sc[t]);
        }
        // reference for the block's exponentials: the max of the fp32-rounded scores
        // (pairs already agree, so the butterfly starts at distance 2)
        mxf = fmaxf(mxf, dpp_f32<kDppXor2>(mxf));
        mxf = fmaxf(mxf, dpp_f32<kDppHalfMirror>(mxf));
        mxf = fmaxf(mxf, dpp_f32<kDppMirror>(mxf));
        mxf = fmaxf(fmaxf(readlane_f32(mxf, 0), readlane_f32(mxf, 16)),
                    fmaxf(readlane_f32(mxf, 32), readlane_f32(mxf, 48)));
        const double mx = (double)mxf;
        // each lane of a pair exponentiates its own half of the pair's tokens
        double sum = 0.0;
#pragma unroll
        for (int tt = 0; tt < NL / 2; ++tt) {
          const long long b0 = __double_as_longlong(sc[2 * tt]), b1 = __double_as_longlong(sc[2 * tt + 1]);
          const double st = __longlong_as_double(half ? b1 : b0);
          sum += (double)fast_exp2((float)((st - mx) * kLog2e));
        }
        sum = wave_sum(sum);
        if (lane == 0) {
          s_mx[j - j0] = mx;
          s_sum[j - j0] = sum;
        }
      }
      if (jn >= j1) break;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NL; ++t) cur[u][t] = nxt[u][t];
      jj = jn;
    }
  }
  __syncthreads();

  // ---- publish e_j = sum_j exp(max_j - M_c) (fp32) and the chunk's (M_c, Z_c = sum_j e_j);
  // the last workgroup of (b, r) to arrive selects
  uint64_t* e_io = blk_e + head * nblk_max;
  if (wave == 0) {
    const int nb = j1 - j0;
    const double x0 = lane < nb ? s_mx[lane] : -INFINITY;
    const double x1 = lane + 64 < nb ? s_mx[lane + 64] : -INFINITY;
    const double mc = wave_max(fmax(x0, x1));
    float e0 = 0.f, e1 = 0.f;
    if (lane < nb) {
      e0 = (float)(s_sum[lane] * (double)fast_exp2((float)((x0 - mc) * kLog2e)));
      st_dev(e_io + j0 + lane, ((uint64_t)__float_as_uint(e0) << 32) | tag);
    }
    if (lane + 64 < nb) {
      e1 = (float)(s_sum[lane + 64] * (double)fast_exp2((float)((x1 - mc) * kLog2e)));
      st_dev(e_io + j0 + lane + 64, ((uint64_t)__float_as_uint(e1) << 32) | tag);
    }
    const double zc = wave_sum((double)e0 + (double)e1);
    if (lane == 0) {
      uint64_t* cs = cmax + (head * n_chunk_max + c) * 2;
      st_dev(cs, tagged(mc, tag));
      st_dev(cs + 1, tagged(zc, tag));
      s_flag = atomicAdd(&counters[head], 1) == nch - 1;
    }
  }
  __syncthreads();
  if (!s_flag) return;

  // ---- M = max_c M_c, Z = sum_c Z_c exp(M_c - M); then m_j = e_j exp(M_c - M) / Z for
  // every block, into LDS
  int budget = kSpinBudget;
  const uint64_t* cs = cmax + head * n_chunk_max * 2;
  if (tid < kBins) {
    sm.bmass[tid] = 0;
    sm.bcnt[tid] = 0;
  }
  if (tid == 0) sm.nfin = 0;
  const int rows = (nblk + kThreads - 1) / kThreads;
  constexpr int LB = 16;  // global reads in flight per thread
  uint64_t w[LB];         // the first LB rows' words go out before the reductions below
#pragma unroll
  for (int u = 0; u < LB; ++u) {
    const int j = u * kThreads + tid;
    w[u] = (u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
  }
  double cm[2], cz[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // nch <= kMaxChunks = 2 * kThreads
    const int i = tid + k * kThreads;
    cm[k] = -INFINITY;
    cz[k] = 0.0;
    if (i < nch) {
      const uint64_t a = ld_dev(cs + 2 * i), z = ld_dev(cs + 2 * i + 1);
      cm[k] = untag(settle(cs + 2 * i, a, tag, budget));
      cz[k] = untag(settle(cs + 2 * i + 1, z, tag, budget));
    }
  }
  const double M = block_reduce(fmax(cm[0], cm[1]), sm.f64, [](double a, double b) { return fmax(a, b); });
  double f[2], zloc = 0.0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    f[k] = cm[k] == -INFINITY ? 0.0 : exp(cm[k] - M);
    zloc += cz[k] * f[k];
  }
  const double invZ = 1.0 / block_reduce(zloc, sm.f64b, SumOp());
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * kThreads;
    if (i < nch) s_f[i] = f[k] * invZ;
  }
  __syncthreads();
  const int cshift = __ffs(chunk_blocks) - 1;
  uint64_t fsum = 0;
  uint32_t bmin = 0xFFFFFFFFu, bmax = 0;
  for (int i0 = 0; i0 < rows; i0 += LB) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int j = (i0 + u) * kThreads + tid;
        w[u] = (i0 + u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
      }
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = (i0 + u) * kThreads + tid;
      if (i0 + u < rows) {
        float m = -1.0f;  // no block
        if (j < nblk) {
          const uint64_t x = settle(e_io + j, w[u], tag, budget);
          m = (float)((double)__uint_as_float((uint32_t)(x >> 32)) * s_f[j >> cshift]);
          fsum += fixed_mass(m);
          bmin = min(bmin, __float_as_uint(m));
          bmax = max(bmax, __float_as_uint(m));
        }
        s_mass[j] = m;
      }
    }
  }
  // one reduction for (sum, min, max)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    fsum += __shfl_xor(fsum, o);
    bmin = min(bmin, (uint32_t)__shfl_xor((int)bmin, o));
    bmax = max(bmax, (uint32_t)__shfl_xor((int)bmax, o));
  }
  if (lane == 0) {
    sm.u64[wave] = fsum;
    sm.u32a[wave] = bmin;
    sm.u32b[wave] = bmax;
  }
  __syncthreads();
  fsum = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    fsum += sm.u64[w2];
    bmin = min(bmin, sm.u32a[w2]);
    bmax = max(bmax, sm.u32b[w2]);
  }

  // threshold key: block j is selected iff key_of(m_j, j) >= thr
  uint64_t thr = 0;
  const float p = top_p[head];
  if (p < 1.0f && nblk > 1) {
    const uint64_t P = (uint64_t)ceil(ldexp((double)p, 62));
    if (fsum >= P)
      thr = select_threshold(s_mass, rows, nblk, P, __builtin_amdgcn_readfirstlane(bmin),
                             __builtin_amdgcn_readfirstlane(bmax), sm);
  }

  // ---- ordered compaction of the selected ids (ascending)
  auto sel = [&](int i, float m) { return m >= 0.f && key_at(i, m) >= thr; };
  const int total = rows_prefix(s_mass, rows, sel, sm);
  int* out = sel_idx + head * nblk_max;
  for_rows(s_mass, rows, [&](int i, float m) {
    const bool sl = sel(i, m);
    const int ord = ordinal(sl, i, sm);
    if (sl) out[ord] = i * kThreads + tid;
  });
  if (tid == 0) {
    sel_cnt[head] = total;
    __hip_atomic_store(&counters[head], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
    __hip_atomic_store(&tags[head], tag % 4095u + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  if (B > 65535 || n_ret > 65535) return RTP_EUNSUPPORTED;
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
  uint32_t* tags = reinterpret_cast<uint32_t*>(ws + L.off_tag);
  uint64_t* cmax = reinterpret_cast<uint64_t*>(ws + L.off_cmax);
  uint64_t* blk_e = reinterpret_cast<uint64_t*>(ws + L.off_e);
  dim3 grid(L.n_chunk, n_ret, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qp = static_cast<const uint16_t*>(q_pre);
  const uint16_t* wq = static_cast<const uint16_t*>(w_q);
  const uint16_t* ki = static_cast<const uint16_t*>(k_idx);
  const size_t dyn = (size_t)L.rows * kThreads * sizeof(float);
  if (block == 64)
    hipLaunchKernelGGL(index_topp_kernel<64>, grid, dim3(kThreads), dyn, s, qp, wq, ki, seq_lens,
                       ret_heads, top_p, Hq, n_ret, max_ctx, L.nblk_max, L.chunk_blocks, L.n_chunk,
                       sel_idx, sel_cnt, counters, tags, cmax, blk_e);
  else
    hipLaunchKernelGGL(index_topp_kernel<128>, grid, dim3(kThreads), dyn, s, qp, wq, ki, seq_lens,
                       ret_heads, top_p, Hq, n_ret, max_ctx, L.nblk_max, L.chunk_blocks, L.n_chunk,
                       sel_idx, sel_cnt, counters, tags, cmax, blk_e);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}
