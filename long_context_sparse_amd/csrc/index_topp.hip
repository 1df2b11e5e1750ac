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
//   is exact and order-independent.  The pass that writes the masses also builds the
//   first 256-bin LDS histogram of (count, mass), half an octave per bin (bits >> 22);
//   one wave scans it for the bin where the cumulative mass from the top crosses p.
//   While more than 64 candidates of unequal mass remain, a further level bins the
//   candidates by (bits - lo) >> shift (>= 128x narrower each time); the last <= 64
//   candidates are gathered (the same pass counts the blocks above them) and ranked
//   exactly by one wave, and a run of equal masses is resolved by count in ascending
//   block order.  The selected ids are written in ascending order by a ballot-based
//   ordered compaction; the arrival counter is reset and the tag advanced.

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
// Mass in fixed point, 2^-62 units, from the bits of a non-negative fp32 mass (< 2):
// floor(m * 2^62) = mantissa * 2^(exponent - 88), truncated.  Integer sums of these are
// exact and independent of order.
__device__ __forceinline__ uint64_t fixed_bits(uint32_t bits) {
  const int e = min((int)(bits >> 23) & 0xFF, 127);
  const uint64_t mant = (bits & 0x7FFFFFu) | 0x800000u;
  if (e >= 88) return mant << (e - 88);
  return e > 64 ? mant >> (88 - e) : 0ull;
}

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
  double f64[kWaves], f64b[kWaves];
  uint64_t ckey[kFinal], cfm[kFinal];  // final candidates (any order)
  uint64_t cab, thr;
  uint32_t lo, hi;
  int cnt, nfin, total, found, ready;
};

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

// One wave: turns rowtab[0 .. rows * kWaves) of per-(row, wave) counts into exclusive
// prefixes in ascending block order and stores their total in sm.total.
__device__ __forceinline__ void rowtab_scan(int rows, TailSmem& sm) {
  const int lane = threadIdx.x & 63;
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

// For a predicate on (row, mass), fills rowtab with the exclusive prefix, in ascending
// block order, of the satisfying blocks per (row, wave) and returns their total; the
// ordinal of a satisfying block is then rowtab[row * kWaves + wave] + (satisfying
// lanes below it in its wave).
template <class Pred>
__device__ __forceinline__ int rows_prefix(const float* __restrict__ sm_m, int rows, Pred pred,
                                           TailSmem& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for_rows(sm_m, rows, [&](int i, float m) {
    const uint64_t bal = __ballot(pred(i, m));
    if (lane == 0) sm.rowtab[i * kWaves + wave] = __popcll(bal);
  });
  __syncthreads();
  if (wave == 0) rowtab_scan(rows, sm);
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

// One wave: scans the bins from the top for the bin where cab + (mass of the bins above
// it) + (its own mass) first reaches P, and records that bin's mass above (sm.cab), count
// (sm.cnt) and bit range [sm.lo, sm.hi]; sets sm.found.  Bin b of a level over [lo, hi]
// holds the bits lo + (b << shift) ..; the top bin also takes everything above.  The bins
// are cleared for the next level.
__device__ __forceinline__ void scan_level(uint64_t cab, uint64_t P, uint32_t lo, uint32_t hi, int shift,
                                           TailSmem& sm) {
  const int lane = threadIdx.x & 63;
  // lane l holds bins kBins-1-4l .. kBins-4-4l (descending mass)
  uint64_t bm[4];
  uint32_t bc[4];
  uint64_t tot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bin = kBins - 1 - 4 * lane - k;
    bm[k] = sm.bmass[bin];
    bc[k] = sm.bcnt[bin];
    tot += bm[k];
    sm.bmass[bin] = 0;
    sm.bcnt[bin] = 0;
  }
  uint64_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  uint64_t run = cab + incl - tot;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (bm[k] > 0 && run < P && run + bm[k] >= P) {
      const uint32_t bin = kBins - 1 - 4 * lane - k;
      const uint32_t blo = lo + (bin << shift);
      sm.cab = run;
      sm.cnt = (int)bc[k];
      sm.lo = blo;
      sm.hi = bin == kBins - 1 ? hi : min(hi, blo + ((1u << shift) - 1u));
      sm.found = 1;
    }
    run += bm[k];
  }
}

__device__ __forceinline__ int level_bin(uint32_t bits, uint32_t lo, int shift) {
  return (int)min((bits - lo) >> shift, (uint32_t)(kBins - 1));
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t a = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t b = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)b << 32) | a;
}

// Exact greedy top-p threshold over the masses in LDS, after a first level whose result
// (sm.cab, sm.cnt, sm.lo, sm.hi) is in place.  Returns the key of the last admitted
// block: the selected set is every block whose key is >= it.  When sm.ready is set on
// return, sm.rowtab already holds the exclusive prefix per (row, wave) of the selected
// blocks and sm.total their number.  Preconditions: the bins and sm.nfin are zero.
//
// Candidates are the blocks whose mass bits lie in [lo, hi], with fixed mass `cab`
// strictly above them, and cab < P <= cab + mass(candidates) holds throughout.  A
// level puts every candidate into one of kBins bins by (bits - lo) >> shift, a
// monotone map, so bins are contiguous ranges of mass (about log-uniform, since fp32
// bits grow with log2 of the value); one wave scans the bins from the top, finds the
// bin where cab + cumulative mass crosses P and takes its bit range as the new candidate
// range (at least kBins/2 times narrower).  It ends when <= kFinal candidates remain
// (ranked exactly by one wave), or when the range is a single mass value: the threshold
// is then the k-th candidate in ascending block order, k = ceil((P - cab) / mass).
__device__ uint64_t select_threshold(const float* __restrict__ sm_m, int rows, uint64_t P, TailSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t cab = uni64(sm.cab);
  int cnt = __builtin_amdgcn_readfirstlane(sm.cnt);
  uint32_t lo = __builtin_amdgcn_readfirstlane(sm.lo);
  uint32_t hi = __builtin_amdgcn_readfirstlane(sm.hi);
  auto cand = [&](float m) {
    const uint32_t bits = __float_as_uint(m);
    return m >= 0.f && bits >= lo && bits <= hi;
  };
  while (cnt > kFinal && lo < hi) {
    const uint32_t span = hi - lo;
    const int shift = max(0, 32 - (int)__clz(span) - 8);  // (span >> shift) < kBins
    for_rows(sm_m, rows, [&](int i, float m) {
      if (cand(m)) {
        const int bin = level_bin(__float_as_uint(m), lo, shift);
        atomicAdd((unsigned long long*)&sm.bmass[bin], (unsigned long long)fixed_bits(__float_as_uint(m)));
        atomicAdd(&sm.bcnt[bin], 1u);
      }
    });
    __syncthreads();
    if (wave == 0) scan_level(cab, P, lo, hi, shift, sm);
    __syncthreads();
    cab = uni64(sm.cab);
    cnt = __builtin_amdgcn_readfirstlane(sm.cnt);
    lo = __builtin_amdgcn_readfirstlane(sm.lo);
    hi = __builtin_amdgcn_readfirstlane(sm.hi);
  }
  if (cnt > kFinal) {
    // every candidate has mass bits lo: admit them in ascending block order
    if (tid == 0) {
      sm.thr = 0;
      sm.ready = 0;
    }
    auto tie = [&](int i, float m) { return m >= 0.f && __float_as_uint(m) == lo; };
    rows_prefix(sm_m, rows, tie, sm);
    const uint64_t f = fixed_bits(lo);
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
  // the last <= kFinal candidates are gathered in any order; the same pass counts, per
  // (row, wave), the blocks above the candidates' range (all selected)
  for_rows(sm_m, rows, [&](int i, float m) {
    const uint32_t bits = __float_as_uint(m);
    if (cand(m)) {
      const int slot = atomicAdd(&sm.nfin, 1);
      if (slot < kFinal) {
        sm.ckey[slot] = key_at(i, m);
        sm.cfm[slot] = fixed_bits(bits);
      }
    }
    const uint64_t bal = __ballot(m >= 0.f && bits > hi);
    if (lane == 0) sm.rowtab[i * kWaves + wave] = __popcll(bal);
  });
  __syncthreads();
  if (wave == 0) {
    // rank by key (keys are distinct): the crossing candidate has cab + (mass of the
    // larger keys) < P <= that + its own mass
    const int nf = min(sm.nfin, kFinal);
    const uint64_t my = lane < nf ? sm.ckey[lane] : 0ull;
    const uint64_t f = lane < nf ? sm.cfm[lane] : 0ull;
    uint64_t above = 0;
    for (int i = 0; i < nf; ++i) {
      const uint64_t ki = readlane_u64(my, i), fi = readlane_u64(f, i);
      above += ki > my ? fi : 0ull;
    }
    const uint64_t cb = __ballot(lane < nf && cab + above < P && cab + above + f >= P);
    const uint64_t thr = cb ? readlane_u64(my, __ffsll((long long)cb) - 1) : 0ull;
    // the selected candidates join the per-(row, wave) counts (LDS operations of one
    // wave complete in order, so the scan below sees them)
    if (cb && lane < nf && my >= thr) {
      const int j = (int)(0xFFFFFFFFu - (uint32_t)my);
      atomicAdd(&sm.rowtab[(j / kThreads) * kWaves + (j % kThreads) / kWave], 1);
    }
    if (cb) rowtab_scan(rows, sm);
    if (lane == 0) {
      sm.thr = thr;
      sm.ready = cb != 0;
      sm.nfin = 0;
    }
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
  if (tid == 0) {
    sm.nfin = 0;
    sm.found = 0;
  }
  const float p = top_p[head];
  const bool pick = p < 1.0f && nblk > 1;  // else every block is selected
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
  {
    const double mw = wave_max(fmax(cm[0], cm[1]));
    if (lane == 0) sm.f64[wave] = mw;
  }
  __syncthreads();
  double M = sm.f64[0];
#pragma unroll
  for (int w2 = 1; w2 < kWaves; ++w2) M = fmax(M, sm.f64[w2]);
  double f[2], zloc = 0.0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    f[k] = cm[k] == -INFINITY ? 0.0 : exp(cm[k] - M);
    zloc += cz[k] * f[k];
  }
  {
    const double zw = wave_sum(zloc);
    if (lane == 0) sm.f64b[wave] = zw;
  }
  __syncthreads();
  double Z = sm.f64b[0];
#pragma unroll
  for (int w2 = 1; w2 < kWaves; ++w2) Z += sm.f64b[w2];
  const double invZ = 1.0 / Z;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * kThreads;
    if (i < nch) s_f[i] = f[k] * invZ;
  }
  __syncthreads();
  // masses into LDS; the same pass builds the first threshold level: 256 bins of half an
  // octave each over the mass bits (bin = bits >> 22, the top bin also takes any larger)
  const int cshift = __ffs(chunk_blocks) - 1;
  for (int i0 = 0; i0 < rows; i0 += LB) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int j = (i0 + u) * kThreads + tid;
        w[u] = (i0 + u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
      }
    }
    bool ok = true;
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = (i0 + u) * kThreads + tid;
      if (i0 + u < rows && j < nblk) ok = ok && (uint32_t)(w[u] & kTagBits) == tag;
    }
    if (!ok) {
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int j = (i0 + u) * kThreads + tid;
        if (i0 + u < rows && j < nblk) w[u] = settle(e_io + j, w[u], tag, budget);
      }
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = (i0 + u) * kThreads + tid;
      if (i0 + u < rows) {
        float m = -1.0f;  // no block
        if (j < nblk) {
          m = (float)((double)__uint_as_float((uint32_t)(w[u] >> 32)) * s_f[j >> cshift]);
          if (pick) {
            const uint32_t bits = __float_as_uint(m);
            const int bin = level_bin(bits, 0u, 22);
            atomicAdd((unsigned long long*)&sm.bmass[bin], (unsigned long long)fixed_bits(bits));
            atomicAdd(&sm.bcnt[bin], 1u);
          }
        }
        s_mass[j] = m;
      }
    }
  }
  __syncthreads();

  // ---- threshold key: block j is selected iff key_of(m_j, j) >= thr
  uint64_t thr = 0;
  bool all = true, ready = false;
  if (pick) {
    const uint64_t P = (uint64_t)ceil(ldexp((double)p, 62));
    if (wave == 0) scan_level(0, P, 0u, 0xFFFFFFFFu, 22, sm);
    __syncthreads();
    if (sm.found) {  // else the total mass is below p: every block
      all = false;
      thr = select_threshold(s_mass, rows, P, sm);
      ready = sm.ready;
    }
  }

  // ---- ordered compaction of the selected ids (ascending)
  int* out = sel_idx + head * nblk_max;
  int total = nblk;
  if (all) {
    for (int j = tid; j < nblk; j += kThreads) out[j] = j;
  } else {
    auto sel = [&](int i, float m) { return m >= 0.f && key_at(i, m) >= thr; };
    total = ready ? sm.total : rows_prefix(s_mass, rows, sel, sm);
    for_rows(s_mass, rows, [&](int i, float m) {
      const bool sl = sel(i, m);
      const int ord = ordinal(sl, i, sm);
      if (sl) out[ord] = i * kThreads + tid;
    });
  }
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
