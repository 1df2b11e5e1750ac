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
//   in fp64.  Per block: lse_j = max + log(sum exp(s - max)).  Per chunk: M_c, Z_c
//   and e_j = exp(lse_j - M_c) go to the workspace.
//   Selection: the last workgroup per (b, r) (device-scope release/acquire around an
//   atomic arrival counter, needed across the 8 XCDs' separate L2s) forms
//   m_j = e_j exp(M_c - M) / Z for every block into LDS and finds the greedy
//   threshold exactly: a key = (fp32 mass bits, inverted block id) orders blocks by
//   mass with ties by ascending id; masses are summed as fixed-point integers (2^-62
//   units) so every cumulative sum is exact and order-independent.  While more than
//   512 candidates remain, 63 evenly spaced candidates are sorted into splitters, a
//   64-bin LDS histogram of (count, mass) over the splitter intervals locates the
//   interval where the cumulative mass crosses p, and that interval becomes the new
//   candidate set; the last <= 512 candidates are ranked exactly and scanned.  The
//   selected ids are written in ascending order by a ballot-based ordered compaction,
//   and the arrival counter is reset to zero.

#include "rtp_common.hpp"

namespace rtp {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunkBlocks = 128;
constexpr int kMaxChunks = 1024;
constexpr int kMaxRows = kThreads / kWaves;   // rows of kThreads blocks in the selection
constexpr int kMaxBlocks = kMaxRows * kThreads;
constexpr int kSplitters = 63;                // splitters per refinement level (64 buckets)
constexpr int kFinal = kThreads;              // candidates ranked directly (one per thread)

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct K1Layout {
  int nblk_max, chunk_blocks, chunk_shift, n_chunk, rows;
  size_t off_counters, off_stats, off_e, total;
};

// Chunk size: aim for >= 1024 workgroups over the whole batch, 8..128 blocks a chunk,
// at most kMaxChunks chunks per head.
K1Layout k1_layout(int B, int n_ret, int max_ctx, int block) {
  K1Layout L{};
  L.nblk_max = ceil_div(max_ctx, block);
  long long total_blocks = (long long)B * n_ret * L.nblk_max;
  int cb = kMaxChunkBlocks;
  while (cb > 8 && total_blocks / cb < 1024) cb >>= 1;
  while (ceil_div(L.nblk_max, cb) > kMaxChunks && cb < kMaxChunkBlocks) cb <<= 1;
  L.chunk_blocks = cb;
  L.chunk_shift = __builtin_ctz(cb);
  L.n_chunk = ceil_div(L.nblk_max, cb);
  L.rows = ceil_div(L.nblk_max, kThreads);
  const size_t heads = (size_t)B * n_ret;
  L.off_counters = 0;
  L.off_stats = align_up(heads * sizeof(int), 256);
  L.off_e = L.off_stats + align_up(heads * L.n_chunk * 2 * sizeof(double), 256);
  L.total = L.off_e + align_up(heads * (size_t)L.nblk_max * sizeof(double), 256);
  return L;
}

// ------------------------------------------------------------------ selection tail
// Composite selection key of block j with fp32 mass m >= 0: the mass bits (order-
// preserving for non-negative floats) above the inverted block id, so that keys are
// distinct and descending key order is descending mass with ties by ascending id.
// Key 0 marks "no block".
__device__ __forceinline__ uint64_t key_of(float m, int j) {
  return ((uint64_t)__float_as_uint(m) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
// Mass in fixed point, 2^-62 units: integer sums are exact and order-independent.
__device__ __forceinline__ uint64_t fixed_mass(float m) { return (uint64_t)((double)m * 0x1p62); }

struct TailSmem {
  uint64_t samp[kSplitters];      // sampled candidate keys
  uint64_t split[kSplitters];     // the same, sorted descending
  uint32_t bcnt[kSplitters + 1];  // per bucket: candidate count
  uint64_t bmass[kSplitters + 1]; // per bucket: fixed-point mass
  int rowtab[kMaxRows * kWaves];  // per (row, wave) counts, then exclusive prefixes
  uint64_t u64[kWaves];
  int i32[kWaves];
  double f64[kWaves];
  uint64_t lo, hi, cab, thr;
  int cnt;
};

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t b = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)b << 32) | a;
}

// Buffers used by one phase at a time.
union PhaseSmem {
  double lse[kMaxChunkBlocks];    // scoring: block lse of this chunk
  double f[kMaxChunks];           // selection: per-chunk factors exp(M_c - M)
  struct {
    uint64_t ckey[kFinal], cfm[kFinal], skey[kFinal], sfm[kFinal];
  } fin;                          // selection: final candidates
};

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over the workgroup; every thread gets the total.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_u64(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

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

// Block j = row * kThreads + thread.  For a predicate on (row), fills rowtab with the
// exclusive prefix, in ascending block order, of the number of blocks satisfying it
// per (row, wave); returns the total.  A caller then gets the ordinal of a satisfying
// block as rowtab[row * kWaves + wave] + (satisfying lanes below it in its wave).
template <class Pred>
__device__ __forceinline__ int rows_prefix(int rows, Pred pred, TailSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll 1
  for (int i = 0; i < rows; ++i) {
    const uint64_t bal = __ballot(pred(i));
    if (lane == 0) sm.rowtab[i * kWaves + wave] = __popcll(bal);
  }
  __syncthreads();
  const int v = tid < rows * kWaves ? sm.rowtab[tid] : 0;
  int total;
  const int excl = block_excl_scan(v, sm.i32, total);
  if (tid < rows * kWaves) sm.rowtab[tid] = excl;
  __syncthreads();
  return total;
}

// Exact greedy top-p threshold over the masses in LDS (mass < 0: no block).  Returns
// the key of the last admitted block: the selected set is every block whose key is
// >= it.  Precondition: the total fixed-point mass reaches P.
//
// Candidates are the keys in [lo, hi) with fixed mass `cab` strictly above them, and
// cab < P <= cab + mass(candidates) holds throughout.  While more than kFinal remain,
// kSplitters candidates evenly spaced in block order are sorted and split the
// candidates into 64 buckets; the bucket where the cumulative mass crosses P becomes
// the new candidate range.  Buckets 0..62 each hold their splitter, so every level
// removes at least 62 candidates.  The last <= kFinal candidates are ranked exactly
// (one per thread) and scanned in descending order.
__device__ __noinline__ uint64_t final_resolve(const float* __restrict__ sm_m, int rows, uint64_t P,
                                                TailSmem& sm, PhaseSmem& ph);

__device__ uint64_t select_threshold(const float* __restrict__ sm_m, int rows, int nblk, uint64_t P,
                                     TailSmem& sm, PhaseSmem& ph) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t lo = 1, hi = ~0ull, cab = 0;
  int cnt = nblk;
  auto key = [&](int i) {
    const float m = sm_m[i * kThreads + tid];
    return m >= 0.f ? key_of(m, i * kThreads + tid) : 0ull;
  };
  while (cnt > kFinal) {
    auto cand = [&](int i) {
      const uint64_t k = key(i);
      return k >= lo && k < hi;
    };
    rows_prefix(rows, cand, sm);
    const int stride = cnt / kSplitters;  // >= 8 since cnt > kFinal
#pragma unroll 1
  for (int i = 0; i < rows; ++i) {
      const uint64_t k = key(i);
      const bool c = k >= lo && k < hi;
      const uint64_t bal = __ballot(c);
      const int ord = sm.rowtab[i * kWaves + wave] + __popcll(bal & lanemask_lt());
      if (c && ord % stride == 0 && ord / stride < kSplitters) sm.samp[ord / stride] = k;
    }
    __syncthreads();
    if (wave == 0) {
      if (lane < kSplitters) {  // rank sort of the (distinct) splitters, descending
        const uint64_t my = sm.samp[lane];
        int rank = 0;
#pragma unroll 1
        for (int i = 0; i < kSplitters; ++i) rank += sm.samp[i] > my ? 1 : 0;
        sm.split[rank] = my;
      }
      sm.bcnt[lane] = 0;
      sm.bmass[lane] = 0;
      if (lane == 0) sm.cnt = 0;
    }
    __syncthreads();
    // bucket of a candidate = number of splitters strictly above its key
#pragma unroll 1
  for (int i = 0; i < rows; ++i) {
      const uint64_t k = key(i);
      if (k >= lo && k < hi) {
        int a = 0, n = kSplitters;  // first index with split[a] <= k
        while (n > 0) {
          const int h = n >> 1;
          if (sm.split[a + h] > k) {
            a += h + 1;
            n -= h + 1;
          } else {
            n = h;
          }
        }
        atomicAdd(&sm.bcnt[a], 1u);
        atomicAdd((unsigned long long*)&sm.bmass[a],
                  (unsigned long long)fixed_mass(sm_m[i * kThreads + tid]));
      }
    }
    __syncthreads();
    if (wave == 0) {
      // bucket b = lane, in descending key order: the one where cab + cumulative mass crosses P
      const uint64_t bm = sm.bmass[lane];
      uint64_t incl = bm;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (cab + incl >= P && cab + incl - bm < P) {
        sm.cab = cab + incl - bm;
        sm.cnt = (int)sm.bcnt[lane];
        sm.hi = lane > 0 ? sm.split[lane - 1] : hi;
        sm.lo = lane < kSplitters ? sm.split[lane] : lo;
      }
    }
    __syncthreads();
    const int nc = __builtin_amdgcn_readfirstlane(sm.cnt);
    if (nc <= 0 || nc >= cnt) {  // cannot happen while the invariant holds; stop safely
      cnt = -1;
      break;
    }
    lo = uni64(sm.lo);
    hi = uni64(sm.hi);
    cab = uni64(sm.cab);
    cnt = __builtin_amdgcn_readfirstlane(nc);
    __syncthreads();
  }
  if (cnt < 0) return 0;  // select every block rather than loop
  if (tid == 0) {
    sm.lo = lo;
    sm.hi = hi;
    sm.cab = cab;
  }
  __syncthreads();
  return final_resolve(sm_m, rows, P, sm, ph);
}

// The last <= kFinal candidates [sm.lo, sm.hi), fixed mass sm.cab above them: gather them
// in block order, rank them exactly, scan in descending order.  A separate function so
// its registers are not live together with the refinement loop's.

__device__ __noinline__ uint64_t final_resolve(const float* __restrict__ sm_m, int rows, uint64_t P,
                                                TailSmem& sm, PhaseSmem& ph) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lo = uni64(sm.lo), hi = uni64(sm.hi), cab = uni64(sm.cab);
  auto key = [&](int i) {
    const float m = sm_m[i * kThreads + tid];
    return m >= 0.f ? key_of(m, i * kThreads + tid) : 0ull;
  };
  auto cand = [&](int i) {
    const uint64_t k = key(i);
    return k >= lo && k < hi;
  };
  const int total = rows_prefix(rows, cand, sm);
#pragma unroll 1
  for (int i = 0; i < rows; ++i) {
    const uint64_t k = key(i);
    const bool c = k >= lo && k < hi;
    const uint64_t bal = __ballot(c);
    const int ord = sm.rowtab[i * kWaves + wave] + __popcll(bal & lanemask_lt());
    if (c && ord < kFinal) {
      ph.fin.ckey[ord] = k;
      ph.fin.cfm[ord] = fixed_mass(sm_m[i * kThreads + tid]);
    }
  }
  if (tid == 0) sm.thr = 0;
  __syncthreads();
  const int nf = total < kFinal ? total : kFinal;
  if (tid < nf) {
    const uint64_t my = ph.fin.ckey[tid];
    int rank = 0;
#pragma unroll 1
    for (int i = 0; i < nf; ++i) rank += ph.fin.ckey[i] > my ? 1 : 0;
    ph.fin.skey[rank] = my;
    ph.fin.sfm[rank] = ph.fin.cfm[tid];
  }
  __syncthreads();
  const uint64_t f = tid < nf ? ph.fin.sfm[tid] : 0ull;
  uint64_t tot64;
  const uint64_t excl = block_excl_scan(f, sm.u64, tot64);
  if (tid < nf && cab + excl < P && cab + excl + f >= P) sm.thr = ph.fin.skey[tid];
  __syncthreads();
  return uni64(sm.thr);
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
  __shared__ PhaseSmem ph;
  __shared__ TailSmem sm;
  __shared__ int s_flag;
  extern __shared__ float s_mass[];   // selection: one fp32 mass per block (rows * kThreads)

  // ---- q_idx = W^Q_r q_pre[b, hq] in fp64 (16 outputs x 16 partial dot products)
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
      if (lane == 0) ph.lse[j - j0] = m + log(sum);
    }
  }
  __syncthreads();

  // ---- chunk epilogue: M_c, Z_c, e_j = exp(lse_j - M_c)
  if (wave == 0) {
    const int nb = j1 - j0;
    const double l0 = lane < nb ? ph.lse[lane] : -INFINITY;
    const double l1 = lane + 64 < nb ? ph.lse[lane + 64] : -INFINITY;
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

  // ---- M, Z and the per-chunk factors exp(M_c - M)
  const double2* st = stats + head * n_chunk_max;
  double mloc = -INFINITY;
  for (int i = tid; i < nch; i += kThreads) mloc = fmax(mloc, st[i].x);
  mloc = wave_max(mloc);
  if (lane == 0) sm.f64[wave] = mloc;
  __syncthreads();
  double M = sm.f64[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmax(M, sm.f64[w]);
  __syncthreads();
  double zloc = 0.0;
  for (int i = tid; i < nch; i += kThreads) {
    const double2 v = st[i];
    const double f = exp(v.x - M);
    ph.f[i] = f;
    zloc += v.y * f;
  }
  zloc = wave_sum(zloc);
  if (lane == 0) sm.f64[wave] = zloc;
  __syncthreads();
  double Z = sm.f64[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) Z += sm.f64[w];
  const double invZ = 1.0 / Z;

  // ---- every block's mass into LDS (block j = row * kThreads + thread), -1 past nblk
  const int rows = (nblk + kThreads - 1) / kThreads;
  const double* eb = blk_e + head * nblk_max;
  uint64_t fsum = 0;
#pragma unroll 1
  for (int i = 0; i < rows; ++i) {
    const int j = i * kThreads + tid;
    const float m = j < nblk ? (float)(eb[j] * (ph.f[j >> chunk_shift] * invZ)) : -1.0f;
    s_mass[j] = m;
    fsum += m > 0.f ? fixed_mass(m) : 0ull;
  }
  __syncthreads();  // ph.f is dead from here on

  // threshold key: block j is selected iff key_of(m_j, j) >= thr
  uint64_t thr = 0;
  const float p = top_p[head];
  if (p < 1.0f && nblk > 1) {
    const uint64_t P = (uint64_t)ceil(ldexp((double)p, 62));
    if (block_sum_u64(fsum, sm.u64) >= P) thr = select_threshold(s_mass, rows, nblk, P, sm, ph);
  }

  // ---- ordered compaction of the selected ids (ascending)
  auto sel = [&](int i) {
    const int j = i * kThreads + tid;
    const float m = s_mass[j];
    return m >= 0.f && key_of(m, j) >= thr;
  };
  const int total = rows_prefix(rows, sel, sm);
  int* out = sel_idx + head * nblk_max;
#pragma unroll 1
  for (int i = 0; i < rows; ++i) {
    const bool sl = sel(i);
    const uint64_t bal = __ballot(sl);
    if (sl) out[sm.rowtab[i * kWaves + wave] + __popcll(bal & lanemask_lt())] = i * kThreads + tid;
  }
  if (tid == 0) {
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
  double2* stats = reinterpret_cast<double2*>(ws + L.off_stats);
  double* blk_e = reinterpret_cast<double*>(ws + L.off_e);
  dim3 grid(L.n_chunk, n_ret, B);
  const size_t dyn = (size_t)L.rows * kThreads * sizeof(float);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qp = static_cast<const uint16_t*>(q_pre);
  const uint16_t* wq = static_cast<const uint16_t*>(w_q);
  const uint16_t* ki = static_cast<const uint16_t*>(k_idx);
  if (block == 64)
    hipLaunchKernelGGL(index_topp_kernel<64>, grid, dim3(kThreads), dyn, s, qp, wq, ki, seq_lens,
                       ret_heads, top_p, Hq, n_ret, max_ctx, L.nblk_max, L.chunk_blocks, L.chunk_shift,
                       L.n_chunk, sel_idx, sel_cnt, counters, stats, blk_e);
  else
    hipLaunchKernelGGL(index_topp_kernel<128>, grid, dim3(kThreads), dyn, s, qp, wq, ki, seq_lens,
                       ret_heads, top_p, Hq, n_ret, max_ctx, L.nblk_max, L.chunk_blocks, L.chunk_shift,
                       L.n_chunk, sel_idx, sel_cnt, counters, stats, blk_e);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}
