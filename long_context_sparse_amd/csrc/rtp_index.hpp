// Device code of kernel 1 (low-rank index scoring and exact block top-p), templated on
// the workgroup size T.
//
// Index score s_n = (W^Q_r q_pre)^T k_idx_n with pre-RoPE features (RTPurbo review,
// Method / Adaptive sparse attention equation); the active set is the block-wise
// top-p of the score distribution, found by a histogram threshold that the last
// workgroup of each head computes, fused with scoring in one launch (review,
// Hardware-aware top-p decoding kernel; "Full Attention Strikes Back" architecture
// paragraph: Kernel 1 at D16, histogram threshold, atomic counters).
//
// Scoring (every workgroup, one chunk of blocks of one (b, r)): each wave streams whole
// KV blocks of the 32 B/token index-key cache with 16-byte loads; one load instruction
// covers 1 KB (32 tokens, two lanes per token).  q_idx and the scores are fp64 so that
// block masses carry < 1e-6 relative error; exponentials are fp32 hardware exp2 on
// arguments already reduced in fp64, summed in fp64; wave reductions run on DPP lane
// moves.  Per block: max_j and sum_j = sum exp(s - max_j); per chunk M_c = max_j max_j,
// and the chunk publishes e_j = sum_j exp(max_j - M_c) (fp32) and (M_c, Z_c) as tagged
// words (rtp_common.hpp), then bumps the head's arrival counter; the last workgroup
// to arrive selects.  So no device-scope fence (an L2 write-back on every workgroup of
// every XCD) is needed, and a word from the previous call is never taken as current.
//
// Selection (last workgroup): M = max_c M_c, Z = sum_c Z_c exp(M_c - M) and every
// block's mass m_j = e_j exp(M_c - M) / Z in fp32 into LDS, then the greedy threshold
// exactly: a key = (fp32 mass bits, inverted block id) orders blocks by mass with ties
// by ascending id; masses are summed as fixed-point integers (2^-62 units) so every
// cumulative sum is exact and order-independent.  Blocks below (1 - p) / (2 nblk) can
// never be selected and stay out; the pass that writes the masses also builds the first
// 256-bin LDS histogram of (count, mass) of the others, an eighth of an octave per bin
// from that floor; one wave scans it for the bin where the cumulative mass from the top
// crosses p.  While more than 64 candidates of unequal mass remain, a further level bins
// the candidates by (bits - lo) >> shift (>= 128x narrower each time); the last <= 64
// candidates are gathered (the same pass counts the blocks above them) and ranked
// exactly by one wave, and a run of equal masses is resolved by count in ascending
// block order.  The selected ids are written in ascending order by a ballot-based
// ordered compaction and the arrival counter is reset.
#pragma once

#include "rtp_common.hpp"

namespace rtp {

constexpr int kIdxMaxChunkBlocks = 256;
constexpr int kIdxMaxBlocks = 16384;            // blocks per sequence the selection holds
constexpr int kBins = 256;                      // histogram bins per refinement level
constexpr int kFinal = kWave;                   // candidates ranked directly (one per lane)
constexpr int kRowTab = kIdxMaxBlocks / kWave;  // (row, wave) entries of the selection
constexpr int kRowBatch = 4;                    // selection rows read together (see for_rows)

template <int T>
struct TailSmem {
  uint64_t bmass[kBins];  // per bin: fixed-point mass
  uint32_t bcnt[kBins];   // per bin: candidate count
  int rowtab[kRowTab];    // per (row, wave) counts, then exclusive prefixes
  double f64[T / kWave], f64b[T / kWave];
  uint64_t above[kFinal];  // final candidates: fixed-point mass of the larger keys
  int wn[T / kWave];       // final candidates gathered by each wave
  uint64_t cab, thr;
  uint32_t lo, hi;
  int cnt, total, found, ready;
};

// LDS of the index role; the per-block masses (rows * T floats) follow it.
template <int T>
struct IndexSmem {
  double qidx[kIndexDim];
  double mx[kIdxMaxChunkBlocks], sum[kIdxMaxChunkBlocks];  // scoring: per-block max, sum
  // selection: per-chunk factor exp(M_c - M) / Z; after the masses are formed, the
  // final candidates each wave gathers (2 * kFinal words a wave)
  double f[2 * T];
  TailSmem<T> sm;
  int flag;
  uint32_t tag;
};
template <int T>
__host__ __device__ constexpr size_t index_smem_bytes(int rows) {
  return (sizeof(IndexSmem<T>) + 15) / 16 * 16 + (size_t)rows * T * sizeof(float);
}
template <int T>
__device__ __forceinline__ float* index_masses(IndexSmem<T>* S) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(S) + (sizeof(IndexSmem<T>) + 15) / 16 * 16);
}

// Chunking of the index role: at least `target` workgroups over the batch where the
// blocks allow, 8..256 blocks (a power of two) a chunk, at most 2 * T chunks per head.  rows = blocks per thread in the selection,
// rounded up to a multiple of kRowBatch.
struct IndexGeom {
  int nblk_max, chunk_blocks, n_chunk, rows;
};
inline IndexGeom index_geom(int B, int n_ret, int max_ctx, int block, int T, int target) {
  IndexGeom g{};
  g.nblk_max = ceil_div(max_ctx, block);
  const long long total_blocks = (long long)B * n_ret * g.nblk_max;
  int cb = kIdxMaxChunkBlocks;
  while (cb > 8 && total_blocks / cb < target) cb >>= 1;
  while (ceil_div(g.nblk_max, cb) > 2 * T && cb < kIdxMaxChunkBlocks) cb <<= 1;
  g.chunk_blocks = cb;
  g.n_chunk = ceil_div(g.nblk_max, cb);
  g.rows = ceil_div(ceil_div(g.nblk_max, T), kRowBatch) * kRowBatch;
  return g;
}

// Global buffers and sizes of the index role.
struct IndexArgs {
  const uint16_t* q_pre;  // bf16 [B, Hq, 128]
  const uint16_t* w_q;    // bf16 [n_ret, 16, 128]
  const uint16_t* k_idx;  // bf16 [B, n_ret, max_ctx, 16]
  const int* seq_lens;
  const int* ret_heads;
  const float* top_p;     // [B * n_ret] top-p of each head (top-p rule)
  int topk_blocks;        // > 0: static top-k, keep this many blocks (top_p unused)
  int Hq, n_ret, max_ctx, nblk_max, chunk_blocks, n_chunk_max;
  int* sel_idx;
  int* sel_cnt;
  uint8_t* sel_mask;  // [B * n_ret, nblk_max] 1 = selected (blocks < nblk), or null
  int* counters;   // [B * n_ret] arrival counters, zero between calls
  uint64_t* cmax;  // [B * n_ret, n_chunk_max, 2] tagged (M_c, Z_c)
  uint64_t* blk_e; // [B * n_ret, nblk_max] tagged e_j
};

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

__device__ __forceinline__ int level_bin(uint32_t bits, uint32_t lo, int shift) {
  return (int)min((bits - lo) >> shift, (uint32_t)(kBins - 1));
}

// Selection rows: block j = row * T + thread, row < rows, masses in LDS (< 0 for no
// block; rows is a multiple of kRowBatch and the rows past the sequence's blocks hold
// -1).  Every pass reads a thread's masses kRowBatch rows at a time, unconditionally,
// so the LDS latencies overlap.
template <int T, class F>
__device__ __forceinline__ void for_rows(const float* __restrict__ sm_m, int rows, F f) {
  const int tid = threadIdx.x;
  for (int i0 = 0; i0 < rows; i0 += kRowBatch) {
    float mm[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) mm[u] = sm_m[(i0 + u) * T + tid];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) f(i0 + u, mm[u]);
  }
}

// A wave's count of a per-row predicate ballot, kept in lane `row` of one register (rows
// <= 64) and stored to rowtab once after the pass.
__device__ __forceinline__ int count_into_lane(int cntv, uint64_t bal, int row) {
  return (int)(threadIdx.x & 63) == row ? (int)__popcll(bal) : cntv;
}
template <int T>
__device__ __forceinline__ void store_row_counts(int cntv, int rows, TailSmem<T>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < rows) sm.rowtab[lane * (T / kWave) + wave] = cntv;
}

// One wave: turns rowtab[0 .. rows * waves) of per-(row, wave) counts into exclusive
// prefixes in ascending block order and stores their total in sm.total.
template <int T>
__device__ __forceinline__ void rowtab_scan(int rows, TailSmem<T>& sm) {
  const int lane = threadIdx.x & 63;
  constexpr int R = kRowTab / 64;  // table entries a lane
  const int n = rows * (T / kWave);
  int v[R], tot = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int idx = lane * R + k;
    v[k] = idx < n ? sm.rowtab[idx] : 0;
    tot += v[k];
  }
  const int incl = (int)wave_incl_scan_u32((uint32_t)tot);
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
// ordinal of a satisfying block is then rowtab[row * waves + wave] + (satisfying
// lanes below it in its wave).
template <int T, class Pred>
__device__ __forceinline__ int rows_prefix(const float* __restrict__ sm_m, int rows, Pred pred,
                                           TailSmem<T>& sm) {
  const int wave = threadIdx.x >> 6;
  int cntv = 0;
  for_rows<T>(sm_m, rows, [&](int i, float m) { cntv = count_into_lane(cntv, __ballot(pred(i, m)), i); });
  store_row_counts<T>(cntv, rows, sm);
  __syncthreads();
  if (wave == 0) rowtab_scan<T>(rows, sm);
  __syncthreads();
  return sm.total;
}

template <int T>
__device__ __forceinline__ int ordinal(bool flag, int i, const TailSmem<T>& sm) {
  const int wave = threadIdx.x >> 6;
  return sm.rowtab[i * (T / kWave) + wave] + __popcll(__ballot(flag) & lanemask_lt());
}

template <int T>
__device__ __forceinline__ uint64_t key_at(int i, float m) {
  return key_of(m, i * T + (int)threadIdx.x);
}

// One wave: scans the bins from the top for the bin where cab + (mass of the bins above
// it) + (its own mass) first reaches P, and records that bin's mass above (sm.cab), count
// (sm.cnt) and bit range [sm.lo, sm.hi]; sets sm.found.  Bin b of a level over [lo, hi]
// holds the bits lo + (b << shift) ..; the top bin also takes everything above.  The bins
// are cleared for the next level.
template <int T>
__device__ __forceinline__ void scan_level(uint64_t cab, uint64_t P, uint32_t lo, uint32_t hi, int shift,
                                           TailSmem<T>& sm) {
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
  const uint64_t incl = wave_incl_scan_u64(tot);
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

// Exact greedy top-p threshold over the masses in LDS, after a first level whose result
// (sm.cab, sm.cnt, sm.lo, sm.hi) is in place.  Returns the key of the last admitted
// block: the selected set is every block whose key is >= it.  When sm.ready is set on
// return, sm.rowtab already holds the exclusive prefix per (row, wave) of the selected
// blocks and sm.total their number.  Preconditions: the bins are zero.  wbuf: LDS for
// the final candidates, 2 * kFinal words per wave.
//
// Candidates are the blocks whose mass bits lie in [lo, hi], with fixed mass `cab`
// strictly above them, and cab < P <= cab + mass(candidates) holds throughout.  A
// level puts every candidate into one of kBins bins by (bits - lo) >> shift, a
// monotone map, so bins are contiguous ranges of mass (about log-uniform, since fp32
// bits grow with log2 of the value); one wave scans the bins from the top, finds the
// bin where cab + cumulative mass crosses P and takes its bit range as the new candidate
// range (at least kBins/2 times narrower).  It ends when <= kFinal candidates remain
// (ranked exactly: every wave compares each candidate with a share of the others), or
// when the range is a single mass value: the threshold is then the k-th candidate in
// ascending block order, k = ceil((P - cab) / mass).
template <int T>
__device__ __noinline__ uint64_t select_threshold(const float* __restrict__ sm_m, int rows, uint64_t P,
                                                  TailSmem<T>& sm, uint64_t* __restrict__ wbuf, bool count) {
  // a block's weight: its fixed-point mass (top-p), or 1 (static top-k: P is then the
  // number of blocks to keep)
  auto wgt = [&](uint32_t bits) { return count ? 1ull : fixed_bits(bits); };
  constexpr int W = T / kWave;
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
    for_rows<T>(sm_m, rows, [&](int i, float m) {
      if (cand(m)) {
        const int bin = level_bin(__float_as_uint(m), lo, shift);
        atomicAdd((unsigned long long*)&sm.bmass[bin], (unsigned long long)wgt(__float_as_uint(m)));
        atomicAdd(&sm.bcnt[bin], 1u);
      }
    });
    __syncthreads();
    if (wave == 0) scan_level<T>(cab, P, lo, hi, shift, sm);
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
    rows_prefix<T>(sm_m, rows, tie, sm);
    const uint64_t f = wgt(lo);
    if (f == 0) return 0;  // cannot happen while the invariant holds
    const uint64_t k = (P - cab + f - 1) / f;  // >= 1, <= cnt
    for_rows<T>(sm_m, rows, [&](int i, float m) {
      const bool c = tie(i, m);
      const int ord = ordinal<T>(c, i, sm);
      if (c && (uint64_t)ord + 1 == k) sm.thr = key_at<T>(i, m);
    });
    __syncthreads();
    return uni64(sm.thr);
  }
  // the last <= kFinal candidates: each wave gathers its own in wbuf (slots from a
  // wave-uniform running count, no atomics); the same pass counts, per (row, wave), the
  // blocks above the candidates' range (all selected)
  uint64_t* wk = wbuf + wave * 2 * kFinal;
  int nw = 0, cntv = 0;
  for_rows<T>(sm_m, rows, [&](int i, float m) {
    const uint32_t bits = __float_as_uint(m);
    const bool c = cand(m);
    const uint64_t bc = __ballot(c);
    if (c) {
      const int slot = nw + (int)__popcll(bc & lanemask_lt());
      if (slot < kFinal) {
        wk[slot] = key_at<T>(i, m);
        wk[kFinal + slot] = wgt(bits);
      }
    }
    nw += (int)__popcll(bc);
    cntv = count_into_lane(cntv, __ballot(m >= 0.f && bits > hi), i);
  });
  store_row_counts<T>(cntv, rows, sm);
  if (lane == 0) sm.wn[wave] = min(nw, kFinal);
  if (wave == 0) sm.above[lane] = 0;
  __syncthreads();
  // every wave holds the candidates one per lane (lane < nf), in wave order
  int nf = 0, sw = 0, sk = 0;
  for (int w2 = 0; w2 < W; ++w2) {
    const int c2 = sm.wn[w2];
    if (lane >= nf && lane < nf + c2) {
      sw = w2;
      sk = lane - nf;
    }
    nf += c2;
  }
  nf = min(nf, kFinal);
  const uint64_t my = lane < nf ? wbuf[sw * 2 * kFinal + sk] : 0ull;
  const uint64_t f = lane < nf ? wbuf[sw * 2 * kFinal + kFinal + sk] : 0ull;
  // rank by key (keys are distinct): wave w sums the masses of the larger keys among
  // candidates w, w + W, ...
  uint64_t part = 0;
  for (int i = wave; i < nf; i += W) {
    const uint64_t ki = readlane_u64(my, i), fi = readlane_u64(f, i);
    part += ki > my ? fi : 0ull;
  }
  if (lane < nf && part) atomicAdd((unsigned long long*)&sm.above[lane], (unsigned long long)part);
  __syncthreads();
  if (wave == 0) {
    // the crossing candidate has cab + (mass of the larger keys) < P <= that + its own
    const uint64_t above = lane < nf ? sm.above[lane] : 0ull;
    const uint64_t cb = __ballot(lane < nf && cab + above < P && cab + above + f >= P);
    const uint64_t thr = cb ? readlane_u64(my, __ffsll((long long)cb) - 1) : 0ull;
    // the selected candidates join the per-(row, wave) counts (LDS operations of one
    // wave complete in order, so the scan below sees them)
    if (cb && lane < nf && my >= thr) {
      const int j = (int)(0xFFFFFFFFu - (uint32_t)my);
      atomicAdd(&sm.rowtab[(j / T) * W + (j % T) / kWave], 1);
    }
    if (cb) rowtab_scan<T>(rows, sm);
    if (lane == 0) {
      sm.thr = thr;
      sm.ready = cb != 0;
    }
  }
  __syncthreads();
  return uni64(sm.thr);
}

// ------------------------------------------------------------------ the index role
// Scores chunk c of head (b, r) and publishes its words; returns true in the workgroup
// that must select (the last of the head to arrive).  The call's tag is read from
// *tag_word and left in S->tag.  Workgroups of chunks past the sequence's end return
// false at once.
template <int BK, int T>
__device__ __forceinline__ bool index_chunk(const IndexArgs& a, int c, int r, int b, const uint32_t* tag_word,
                                            IndexSmem<T>* S) {
  static_assert(T >= 256 && T % kWave == 0, "the q_idx product and the bins take 256 threads");
  constexpr int W = T / kWave;
  constexpr int NL = BK / 32;          // 1 KB loads per lane per block
  constexpr int U = BK == 64 ? 2 : 1;  // blocks in flight per wave
  const int N = a.seq_lens[b];
  const int nblk = (N + BK - 1) / BK;
  const int nch = (nblk + a.chunk_blocks - 1) / a.chunk_blocks;
  if (c >= nch) return false;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head = (size_t)b * a.n_ret + r;

  // ---- scoring: max and sum of every block of this chunk into LDS.  Wave w takes blocks
  // j0 + w + W * (U * k + u); the next U blocks' loads are in flight while the current U
  // blocks are reduced.
  const int half = lane & 1;
  const uint16_t* kb = a.k_idx + head * (size_t)a.max_ctx * kIndexDim + half * 8;
  const int j0 = c * a.chunk_blocks;
  const int j1 = min(j0 + a.chunk_blocks, nblk);
  // Every load is unconditional and streaming (the keys are read once): a token past the
  // sequence's end (or of a block past the chunk's end) reads token `last` instead and its
  // score is masked (or the block skipped) below.  Branch-free loads let the compiler
  // count them, so the next blocks' loads stay in flight while the current ones are
  // reduced.
  auto load = [&](uint4 (&v)[U][NL], int jj, int last) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jj + u * W;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int tok = min(j * BK + 32 * t + (lane >> 1), last);
        v[u][t] = ld16_nt(kb + (size_t)tok * kIndexDim);
      }
    }
  };
  // the first blocks' loads go out before q_idx is formed
  int jj = j0 + wave;
  uint4 cur[U][NL];
  if (jj < j1) load(cur, jj, N - 1);

  // ---- this call's tag; q_idx = W^Q_r q_pre[b, hq] in fp64 (16 outputs x 16 partial dots)
  if (tid == 0) S->tag = load_tag(tag_word);
  if (tid < 256) {
    const int hq = a.ret_heads[r];
    const int i = tid >> 4, part = tid & 15;
    const uint4 wv = ld16(a.w_q + ((size_t)r * kIndexDim + i) * kHeadDim + part * 8);
    const uint4 qv = ld16(a.q_pre + ((size_t)b * a.Hq + hq) * kHeadDim + part * 8);
    double x = (double)bf_lo(wv.x) * (double)bf_lo(qv.x);
    x = fma((double)bf_hi(wv.x), (double)bf_hi(qv.x), x);
    x = fma((double)bf_lo(wv.y), (double)bf_lo(qv.y), x);
    x = fma((double)bf_hi(wv.y), (double)bf_hi(qv.y), x);
    x = fma((double)bf_lo(wv.z), (double)bf_lo(qv.z), x);
    x = fma((double)bf_hi(wv.z), (double)bf_hi(qv.z), x);
    x = fma((double)bf_lo(wv.w), (double)bf_lo(qv.w), x);
    x = fma((double)bf_hi(wv.w), (double)bf_hi(qv.w), x);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o);
    if (part == 0) S->qidx[i] = x;
  }
  __syncthreads();
  const uint32_t tag = S->tag;
  double qh[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) qh[k] = S->qidx[half * 8 + k];

  if (jj < j1) {
    while (true) {
      const int jn = jj + W * U;
      uint4 nxt[U][NL];
      // past the chunk's end every lane reads the current block's first token (32 B)
      load(nxt, jn < j1 ? jn : jj, jn < j1 ? N - 1 : jj * BK);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jj + u * W;
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
          double s = a0 + a1;
          s += dpp_f64<kDppXor1>(s);  // commutative: both lanes of the pair get the same value
          const int tok = j * BK + 32 * t + (lane >> 1);
          sc[t] = tok < N ? s : -INFINITY;
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
          S->mx[j - j0] = mx;
          S->sum[j - j0] = sum;
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
  uint64_t* e_io = a.blk_e + head * a.nblk_max;
  if (wave == 0) {
    constexpr int PL = kIdxMaxChunkBlocks / kWave;  // blocks of the chunk per lane
    const int nb = j1 - j0;
    double x[PL];
    double xm = -INFINITY;
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      x[q] = lane + kWave * q < nb ? S->mx[lane + kWave * q] : -INFINITY;
      xm = fmax(xm, x[q]);
    }
    const double mc = wave_max(xm);
    double zl = 0.0;
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int k = lane + kWave * q;
      if (k < nb) {
        const float e = (float)(S->sum[k] * (double)fast_exp2((float)((x[q] - mc) * kLog2e)));
        st_dev(e_io + j0 + k, tagged_f32(e, tag));
        zl += (double)e;
      }
    }
    const double zc = wave_sum(zl);
    if (lane == 0) {
      uint64_t* cs = a.cmax + (head * a.n_chunk_max + c) * 2;
      st_dev(cs, tagged(mc, tag));
      st_dev(cs + 1, tagged(zc, tag));
      S->flag = atomicAdd(&a.counters[head], 1) == nch - 1;
    }
  }
  __syncthreads();
  return S->flag != 0;
}

// The selection of head (b, r), run by the workgroup index_chunk picked: writes the
// ascending selected block ids and their count (and, if asked, one byte per block:
// 1 = selected), and resets the head's arrival counter.
template <int T>
__device__ __forceinline__ void index_select(const IndexArgs& a, int BK, int r, int b, IndexSmem<T>* S) {
  constexpr int W = T / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head = (size_t)b * a.n_ret + r;
  const int N = a.seq_lens[b];
  const int nblk = (N + BK - 1) / BK;
  const int nch = (nblk + a.chunk_blocks - 1) / a.chunk_blocks;
  const uint32_t tag = S->tag;
  TailSmem<T>& sm = S->sm;
  float* s_mass = index_masses<T>(S);
  const uint64_t* e_io = a.blk_e + head * a.nblk_max;

  // ---- M = max_c M_c, Z = sum_c Z_c exp(M_c - M); then m_j = e_j exp(M_c - M) / Z for
  // every block, into LDS
  int budget = kSpinBudget;
  const uint64_t* cs = a.cmax + head * a.n_chunk_max * 2;
  if (tid < kBins) {
    sm.bmass[tid] = 0;
    sm.bcnt[tid] = 0;
  }
  if (tid == 0) sm.found = 0;
  // static top-k keeps topk_blocks blocks: the same search with every block weighing 1
  // and P = the number of blocks
  const int kb = a.topk_blocks;
  const bool count = kb > 0;
  const float p = count ? 1.0f : a.top_p[head];
  const bool pick = count ? kb < nblk : (p < 1.0f && nblk > 1);  // else every block is selected
  // Top-p: every block of mass below (1 - p) / (2 nblk) is outside the selection and
  // below its threshold: with total mass ~1 the threshold exceeds (total - p) / nblk.
  // Such blocks stay out of the histograms (peaked heads have thousands of them).
  const uint32_t lbits = count ? 0u : __float_as_uint(fmaxf(0.f, 0.5f * (1.0f - p - 1e-6f) / (float)nblk));
  // first level: 1/8-octave bins (bits >> 20) from the floor up, which span 32 octaves
  // (everything above goes to the top bin); without a floor, half-octave bins from 0
  const int shift1 = lbits ? 20 : 22;
  const uint32_t lo1 = lbits & ~((1u << shift1) - 1u);
  const int rows = ceil_div(ceil_div(nblk, T), kRowBatch) * kRowBatch;  // rows past nblk hold -1
  constexpr int LB = 16;  // global reads in flight per thread
  uint64_t w[LB];         // the first LB rows' words go out before the reductions below
#pragma unroll
  for (int u = 0; u < LB; ++u) {
    const int j = u * T + tid;
    w[u] = (u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
  }
  double cm[2], cz[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // nch <= 2 * T
    const int i = tid + k * T;
    cm[k] = -INFINITY;
    cz[k] = 0.0;
    if (i < nch) {
      const uint64_t x = ld_dev(cs + 2 * i), z = ld_dev(cs + 2 * i + 1);
      cm[k] = untag(settle(cs + 2 * i, x, tag, budget));
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
  for (int w2 = 1; w2 < W; ++w2) M = fmax(M, sm.f64[w2]);
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
  for (int w2 = 1; w2 < W; ++w2) Z += sm.f64b[w2];
  const double invZ = 1.0 / Z;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = tid + k * T;
    if (i < nch) S->f[i] = f[k] * invZ;
  }
  __syncthreads();
  // masses into LDS; the same pass builds the first threshold level over the blocks above
  // the floor: bin = (bits - lo1) >> shift1, the top bin also takes any larger
  const int cshift = __ffs(a.chunk_blocks) - 1;
  for (int i0 = 0; i0 < rows; i0 += LB) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int j = (i0 + u) * T + tid;
        w[u] = (i0 + u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
      }
    }
    bool ok = true;
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = (i0 + u) * T + tid;
      if (i0 + u < rows && j < nblk) ok = ok && has_tag(w[u], tag);
    }
    if (!ok) {
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int j = (i0 + u) * T + tid;
        if (i0 + u < rows && j < nblk) w[u] = settle(e_io + j, w[u], tag, budget);
      }
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int j = (i0 + u) * T + tid;
      if (i0 + u < rows) {
        float m = -1.0f;  // no block
        if (j < nblk) {
          m = (float)((double)untag_f32(w[u]) * S->f[j >> cshift]);
          const uint32_t bits = __float_as_uint(m);
          if (pick && bits >= lbits) {
            const int bin = level_bin(bits, lo1, shift1);
            atomicAdd((unsigned long long*)&sm.bmass[bin], count ? 1ull : (unsigned long long)fixed_bits(bits));
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
    const uint64_t P = count ? (uint64_t)kb : (uint64_t)ceil(ldexp((double)p, 62));
    if (wave == 0) {
      scan_level<T>(0, P, lo1, 0xFFFFFFFFu, shift1, sm);
      // the pruned blocks were not counted: the candidates start at the floor
      if (lane == 0 && sm.found) sm.lo = min(max(sm.lo, lbits), sm.hi);
    }
    __syncthreads();
    if (sm.found) {  // else the total mass is below p: every block
      all = false;
      thr = select_threshold<T>(s_mass, rows, P, sm, reinterpret_cast<uint64_t*>(S->f), count);
      ready = sm.ready;
    }
  }

  // ---- ordered compaction of the selected ids (ascending)
  int* out = a.sel_idx + head * a.nblk_max;
  uint8_t* mask = a.sel_mask ? a.sel_mask + head * a.nblk_max : nullptr;
  int total = nblk;
  if (all) {
    for (int j = tid; j < nblk; j += T) {
      out[j] = j;
      if (mask) mask[j] = 1;
    }
  } else {
    auto sel = [&](int i, float m) { return m >= 0.f && key_at<T>(i, m) >= thr; };
    total = ready ? sm.total : rows_prefix<T>(s_mass, rows, sel, sm);
    for_rows<T>(s_mass, rows, [&](int i, float m) {
      const bool sl = sel(i, m);
      const int ord = ordinal<T>(sl, i, sm);
      const int j = i * T + tid;
      if (sl) out[ord] = j;
      if (mask && j < nblk) mask[j] = sl;
    });
  }
  if (tid == 0) {
    a.sel_cnt[head] = total;
    __hip_atomic_store(&a.counters[head], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
  }
}

}  // namespace rtp
