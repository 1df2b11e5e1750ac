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
// and the chunk publishes e_j = sum_j exp(max_j - M_c) and (M_c, Z_c) as tagged fp32
// words (rtp_common.hpp), then bumps the head's arrival counter; the last workgroup
// to arrive selects.  So no device-scope fence (an L2 write-back on every workgroup of
// every XCD) is needed, and a word from an earlier call is never taken as current.  A
// selecting workgroup whose bounded wait for a word runs out selects every block of its
// head (a superset of the top-p set) and reports it in the workspace header.
//
// Workspace: a header (layout key, sticky status bits, fallback count, a fault-injection
// word for tests), then one region per (sequence, retrieval head) at a stride that
// depends only on the blocks per sequence: the head's arrival counter and tag, its chunk
// words, its block words and its chunks' heavy-block lists.  Calls with other batch sizes or head counts reuse it; a
// call whose blocks per sequence differ from the layout the workspace was first used
// with is refused on the device (every block selected, status bit set).
//
// Selection (last workgroup): M = max_c M_c, Z = sum_c Z_c exp(M_c - M) and every
// block's mass m_j = e_j exp(M_c - M) / Z in fp32 into LDS, then the greedy threshold
// exactly: a key = (fp32 mass bits, inverted block id) orders blocks by mass with ties
// by ascending id; masses are summed as fixed-point integers (2^-62 units) so every
// cumulative sum is exact and order-independent.  Blocks below (1 - p) / (2 nblk) can
// never be selected and stay out; the pass that writes the masses gathers the others into
// a candidate list (one LDS atomic per wave and row) and builds the first 256-bin LDS
// histogram of (count, mass) of them, an eighth of an octave per bin from that floor; one
// wave scans it for the bin where the cumulative mass from the top crosses p.  While more
// than 64 candidates of unequal mass remain, a further level bins the candidates of the
// crossing range by (bits - lo) >> shift (>= 128x narrower each time); the last <= 64 are
// gathered and ranked exactly, and a run of equal masses is resolved by count in
// ascending block order (found on an LDS bitmap).  Every pass after the masses runs over
// the candidate list only (a handful of blocks for a peaked head).  The selected ids are
// written in ascending order from an LDS bitmap of the selected blocks (a prefix count of
// its words gives each block its slot) and the arrival counter is reset.
#pragma once

#include "rtp_common.hpp"

namespace rtp {

constexpr int kIdxMaxChunkBlocks = 256;
constexpr int kIdxMaxBlocks = 16384;             // blocks per sequence the selection holds
constexpr int kIdxMaxChunks = 2048;              // chunks per head the selection combines
constexpr int kBins = 256;                       // histogram bins per refinement level
constexpr int kFinal = kWave;                    // candidates ranked directly (one per lane)
constexpr int kBitWords = kIdxMaxBlocks / 32;    // words of a block bitmap
constexpr int kMassBatch = 8;                    // block words a thread loads before using them
constexpr int kListSlots = 8;                    // heavy blocks a chunk lists (e_j >= Z_c / 8)
constexpr int kListWords = 1 + 2 * kListSlots;   // a chunk's list: its count, then (e_j, j) pairs
constexpr int kListMaxChunks = 128;              // chunks per head that publish lists

constexpr int kBitWordsPerLane = kBitWords / kWave;  // bitmap words a lane of one wave scans

struct TailSmem {
  uint64_t bmass[kBins];        // per bin: fixed-point mass
  uint32_t bcnt[kBins];         // per bin: candidate count
  uint32_t sel[kBitWords];      // bitmap of the selected blocks
  uint32_t tie[kBitWords];      // bitmap of the candidates of one tied mass
  uint32_t wpre[kBitWords];     // exclusive prefix of the bitmap words' bit counts
  uint64_t fkey[kFinal], fw[kFinal];  // the last <= kFinal candidates: keys and weights
  uint64_t cab, thr;
  uint32_t lo, hi;
  int cnt, found, ncand, nfinal, total;
  // the chunks' heavy-block lists: counts, fp32 Z_c, the bound on every unlisted block's
  // mass (fp32 bits), the listed blocks, those gathered above the bound, a list
  // overflowed or a wait ran out, the lists decided
  int lcnt[kListMaxChunks];
  float lz[kListMaxChunks];
  uint32_t ubound;
  int nlist, ngath, lbad, lok;
};

// LDS of the index role; the per-block masses (rows * T floats) and the candidate list
// (rows * T block ids) follow it.
template <int T>
struct IndexSmem {
  double qidx[kIndexDim];
  double mx[kIdxMaxChunkBlocks], sum[kIdxMaxChunkBlocks];  // scoring: per-block max, sum
  // selection: the chunk words (M_c, Z_c as fp32), then the chunk factors exp(M_c - M) / Z
  // (fp32); after the masses are formed, the final candidates each wave gathers (2 *
  // kFinal words a wave)
  float cm[kIdxMaxChunks], cz[kIdxMaxChunks];
  TailSmem sm;
  int flag;
  uint32_t tag;
  int inject, mismatch;
};
template <int T>
__host__ __device__ constexpr size_t index_smem_bytes(int rows) {
  return (sizeof(IndexSmem<T>) + 15) / 16 * 16 + (size_t)rows * T * (sizeof(float) + sizeof(uint16_t));
}
template <int T>
__device__ __forceinline__ float* index_masses(IndexSmem<T>* S) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(S) + (sizeof(IndexSmem<T>) + 15) / 16 * 16);
}
template <int T>
__device__ __forceinline__ uint16_t* index_cands(IndexSmem<T>* S, int rows) {
  return reinterpret_cast<uint16_t*>(index_masses<T>(S) + (size_t)rows * T);
}

// Chunking of the index role: at least `target` workgroups over the batch where the
// blocks allow, 8..256 blocks (a power of two) a chunk, at most 2 * T chunks per head.
// rows = blocks per thread in the selection.
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
  g.rows = ceil_div(g.nblk_max, T);
  return g;
}

// Index workspace layout (see the file comment): the header, then per head a 256-byte
// state record (arrival counter, tag) followed by 2 words per chunk (M_c, Z_c), one
// word per block (e_j) and, for the first 128 chunks, a list of kListWords words (the
// count of blocks with e_j >= Z_c / 8, then up to 8 (e_j, j) pairs).  Chunks hold >= 8
// blocks, so a head has at most min(2048, ceil(nblk_max / 8)) chunks.
struct IndexWsHeader {
  uint32_t layout;     // blocks per sequence of the calls this workspace serves (0: fresh)
  uint32_t status;     // sticky error bits (RTP_INDEX_WAIT_EXPIRED, RTP_INDEX_LAYOUT_MISMATCH)
  uint32_t fallbacks;  // selections that fell back to every block
  uint32_t inject;     // bit 0: every bounded wait gives up at once (failure-path tests)
};
struct IndexHeadState {
  int counter;   // arrival counter, zero between calls
  uint32_t tag;  // tag of the head's next call (0 in a fresh workspace reads as 1)
};
constexpr size_t kIdxWsHeaderBytes = 256;
constexpr size_t kIdxHeadStateBytes = 256;

__host__ __device__ inline int index_chunk_cap(int nblk_max) {
  const int c = (nblk_max + 7) / 8;
  return c < kIdxMaxChunks ? c : kIdxMaxChunks;
}
__host__ __device__ inline int index_list_cap(int nblk_max) {
  const int c = index_chunk_cap(nblk_max);
  return c < kListMaxChunks ? c : kListMaxChunks;
}
__host__ __device__ inline size_t index_head_stride(int nblk_max) {
  return align_up(kIdxHeadStateBytes + (size_t)index_chunk_cap(nblk_max) * 16 + (size_t)nblk_max * 8 +
                      (size_t)index_list_cap(nblk_max) * kListWords * 8,
                  256);
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
  int Hq, n_ret, max_ctx, nblk_max, chunk_blocks, n_chunk_cap;
  int* sel_idx;
  int* sel_cnt;
  uint8_t* sel_mask;  // [B * n_ret, nblk_max] 1 = selected (blocks < nblk), or null
  IndexWsHeader* hdr;
  char* regions;       // per-head regions, head_stride bytes apart
  size_t head_stride;
};
__device__ __forceinline__ IndexHeadState* head_state(const IndexArgs& a, size_t head) {
  return reinterpret_cast<IndexHeadState*>(a.regions + head * a.head_stride);
}
__device__ __forceinline__ uint64_t* head_chunk_words(const IndexArgs& a, size_t head) {
  return reinterpret_cast<uint64_t*>(a.regions + head * a.head_stride + kIdxHeadStateBytes);
}
__device__ __forceinline__ uint64_t* head_block_words(const IndexArgs& a, size_t head) {
  return head_chunk_words(a, head) + 2 * (size_t)a.n_chunk_cap;
}
__device__ __forceinline__ uint64_t* head_list_words(const IndexArgs& a, size_t head) {
  return head_block_words(a, head) + (size_t)a.nblk_max;
}
// Whether a head's chunks publish heavy-block lists and its selection tries them first:
// top-p, at most kListMaxChunks chunks, and more than two rows of blocks a thread (below
// that the full mass pass is short and the lists do not repay their words).
__device__ __forceinline__ bool index_lists(const IndexArgs& a, int nblk, int nch, int T) {
  return a.topk_blocks == 0 && nch <= kListMaxChunks && nblk > 2 * T;
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

__device__ __forceinline__ int level_bin(uint32_t bits, uint32_t lo, int shift) {
  return (int)min((bits - lo) >> shift, (uint32_t)(kBins - 1));
}

// One wave: exclusive prefix of the bit counts of bitmap words [0, nwords) (consecutive
// words per lane) into sm.wpre, their total into sm.total.
__device__ __forceinline__ void bitmap_prefix_wave(const uint32_t* __restrict__ bits, int nwords, TailSmem& sm) {
  const int lane = threadIdx.x & 63;
  uint32_t c[kBitWordsPerLane], v = 0;
#pragma unroll
  for (int k = 0; k < kBitWordsPerLane; ++k) {
    const int i = lane * kBitWordsPerLane + k;
    c[k] = i < nwords ? (uint32_t)__popc(bits[i]) : 0u;
    v += c[k];
  }
  const uint32_t incl = wave_incl_scan_u32(v);
  uint32_t off = incl - v;
#pragma unroll
  for (int k = 0; k < kBitWordsPerLane; ++k) {
    const int i = lane * kBitWordsPerLane + k;
    if (i < nwords) sm.wpre[i] = off;
    off += c[k];
  }
  if (lane == 63) sm.total = (int)incl;
}

// Slot of block j among the set bits of a bitmap whose word prefixes are in sm.wpre.
__device__ __forceinline__ int bitmap_rank(const uint32_t* __restrict__ bits, int j, const TailSmem& sm) {
  return (int)sm.wpre[j >> 5] + __popc(bits[j >> 5] & ((1u << (j & 31)) - 1u));
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

// Exact greedy top-p threshold over the candidates cand[0, nc) (their masses in sm_m),
// after a first level whose result (sm.cab, sm.cnt, sm.lo, sm.hi) is in place.  Returns
// the key of the last admitted block: the selected set is every candidate whose key is
// >= it.  Passes over the candidates run on all T threads; scans and the final ranking on
// wave 0 alone (the other waves wait at the barrier, issuing nothing).  Preconditions:
// the bins, sm.tie and sm.nfinal are zero.
//
// Candidates of a level are those whose mass bits lie in [lo, hi], with fixed mass `cab`
// strictly above them, and cab < P <= cab + mass(candidates) holds throughout.  A level
// puts every candidate into one of kBins bins by (bits - lo) >> shift, a monotone map, so
// bins are contiguous ranges of mass (about log-uniform, since fp32 bits grow with log2
// of the value); one wave scans the bins from the top, finds the bin where cab +
// cumulative mass crosses P and takes its bit range as the new range (at least kBins/2
// times narrower).  It ends when <= kFinal candidates remain (ranked exactly by one wave,
// one candidate a lane), or when the range is a single mass value: the threshold is then
// the k-th candidate in ascending block order, k = ceil((P - cab) / mass).  V tells
// kernel builds with different register budgets apart, so each gets its own copy.
template <int T, int V>
__device__ __noinline__ uint64_t select_threshold(const float* __restrict__ sm_m, const uint16_t* __restrict__ cand,
                                                  int nc, int nblk, uint64_t P, TailSmem& sm, bool count) {
  // a block's weight: its fixed-point mass (top-p), or 1 (static top-k: P is then the
  // number of blocks to keep)
  auto wgt = [&](uint32_t bits) { return count ? 1ull : fixed_bits(bits); };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t cab = uni64(sm.cab);
  int cnt = __builtin_amdgcn_readfirstlane(sm.cnt);
  uint32_t lo = __builtin_amdgcn_readfirstlane(sm.lo);
  uint32_t hi = __builtin_amdgcn_readfirstlane(sm.hi);
  while (cnt > kFinal && lo < hi) {
    const uint32_t span = hi - lo;
    const int shift = max(0, 32 - (int)__clz(span) - 8);  // (span >> shift) < kBins
    for (int k = tid; k < nc; k += T) {
      const uint32_t bits = __float_as_uint(sm_m[cand[k]]);
      if (bits >= lo && bits <= hi) {
        const int bin = level_bin(bits, lo, shift);
        atomicAdd((unsigned long long*)&sm.bmass[bin], (unsigned long long)wgt(bits));
        atomicAdd(&sm.bcnt[bin], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) scan_level(cab, P, lo, hi, shift, sm);
    __syncthreads();
    cab = uni64(sm.cab);
    cnt = __builtin_amdgcn_readfirstlane(sm.cnt);
    lo = __builtin_amdgcn_readfirstlane(sm.lo);
    hi = __builtin_amdgcn_readfirstlane(sm.hi);
  }
  if (cnt > kFinal) {
    // every candidate left has mass bits lo: admit them in ascending block order, the
    // k-th of them found on a bitmap of the tied blocks
    if (tid == 0) sm.thr = 0;
    for (int k = tid; k < nc; k += T) {
      const int j = cand[k];
      if (__float_as_uint(sm_m[j]) == lo) atomicOr(&sm.tie[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    if (wave == 0) {
      const int nwords = ceil_div(nblk, 32);
      bitmap_prefix_wave(sm.tie, nwords, sm);
      const uint64_t f = wgt(lo);
      const uint32_t kk = (uint32_t)(f ? (P - cab + f - 1) / f : 1);  // >= 1, <= cnt
      // the word holding the kk-th tied block, then the bit within it
#pragma unroll
      for (int q = 0; q < kBitWordsPerLane; ++q) {
        const int i = lane * kBitWordsPerLane + q;
        if (i < nwords) {
          uint32_t word = sm.tie[i];
          const uint32_t before = sm.wpre[i];
          if (before < kk && kk <= before + (uint32_t)__popc(word)) {
            for (uint32_t r = kk - before; r > 1; --r) word &= word - 1u;  // drop the lower bits
            sm.thr = key_of(__uint_as_float(lo), i * 32 + __ffs(word) - 1);
          }
        }
      }
    }
    __syncthreads();
    return uni64(sm.thr);
  }
  // the last <= kFinal candidates: appended to one short list, then ranked by wave 0
  for (int k = tid; k < nc; k += T) {
    const int j = cand[k];
    const uint32_t bits = __float_as_uint(sm_m[j]);
    if (bits >= lo && bits <= hi) {
      const int slot = atomicAdd(&sm.nfinal, 1);
      if (slot < kFinal) {
        sm.fkey[slot] = key_of(__uint_as_float(bits), j);
        sm.fw[slot] = wgt(bits);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int nf = min(sm.nfinal, kFinal);
    const uint64_t my = lane < nf ? sm.fkey[lane] : 0ull;
    const uint64_t f = lane < nf ? sm.fw[lane] : 0ull;
    // rank by key (keys are distinct): the mass of the larger keys
    uint64_t above = 0;
    for (int i = 0; i < nf; ++i) {
      const uint64_t ki = readlane_u64(my, i), fi = readlane_u64(f, i);
      above += ki > my ? fi : 0ull;
    }
    // the crossing candidate has cab + (mass of the larger keys) < P <= that + its own
    const uint64_t cb = __ballot(lane < nf && cab + above < P && cab + above + f >= P);
    const uint64_t thr = cb ? readlane_u64(my, __ffsll((long long)cb) - 1) : 0ull;
    if (lane == 0) sm.thr = thr;
  }
  __syncthreads();
  return uni64(sm.thr);
}

// ------------------------------------------------------------------ the index role
// Every block of head (b, r) selected (blocks < nblk): the list 0 .. nblk - 1, its count
// and the mask.  The fallback of a selection that cannot run.
template <int T>
__device__ __forceinline__ void select_all(const IndexArgs& a, size_t head, int nblk) {
  int* out = a.sel_idx + head * a.nblk_max;
  uint8_t* mask = a.sel_mask ? a.sel_mask + head * a.nblk_max : nullptr;
  for (int j = threadIdx.x; j < nblk; j += T) {
    out[j] = j;
    if (mask) mask[j] = 1;
  }
  if (threadIdx.x == 0) a.sel_cnt[head] = nblk;
}

// Scores chunk c of head (b, r) and publishes its words; returns true in the workgroup
// that must select (the last of the head to arrive).  The call's tag is read from the
// head's state and left in S->tag.  Workgroups of chunks past the sequence's end return
// false at once.  When the workspace was laid out for another number of blocks per
// sequence, nothing of it is touched: chunk 0 selects every block of the head and sets
// the header's status bit, and every workgroup returns false.
template <int BK, int T>
__device__ __forceinline__ bool index_chunk(const IndexArgs& a, int c, int r, int b, IndexSmem<T>* S) {
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

  // ---- this call's tag and the workspace's layout key; q_idx = W^Q_r q_pre[b, hq] in
  // fp64 (16 outputs x 16 partial dots)
  if (tid == 0) {
    S->tag = load_tag(&head_state(a, head)->tag);
    const uint32_t lay = __hip_atomic_load(&a.hdr->layout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S->inject = (int)__hip_atomic_load(&a.hdr->inject, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S->mismatch = lay != 0u && lay != (uint32_t)a.nblk_max;
    if (lay == 0u && c == 0)  // a fresh workspace takes this call's layout
      __hip_atomic_store(&a.hdr->layout, (uint32_t)a.nblk_max, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
  if (S->mismatch) {
    if (c == 0) {
      select_all<T>(a, head, nblk);
      if (tid == 0) {
        atomicOr(&a.hdr->status, (uint32_t)RTP_INDEX_LAYOUT_MISMATCH);
        atomicAdd(&a.hdr->fallbacks, 1u);
      }
    }
    return false;
  }
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
  uint64_t* e_io = head_block_words(a, head);
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
    float ev[PL];  // -1: no block
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int k = lane + kWave * q;
      ev[q] = -1.0f;
      if (k < nb) {
        const float e = (float)(S->sum[k] * (double)fast_exp2((float)((x[q] - mc) * kLog2e)));
        st_dev(e_io + j0 + k, tagged_f32(e, tag));
        zl += (double)e;
        ev[q] = e;
      }
    }
    const double zc = wave_sum(zl);
    // the chunk's heavy blocks (e_j >= Z_c / 8 in fp32, so at most 8 unless Z_c is
    // degenerate), ascending, and their count; the selection may decide from these lists
    // alone (index_select)
    if (index_lists(a, nblk, nch, T)) {
      uint64_t* lw = head_list_words(a, head) + (size_t)c * kListWords;
      const float lim = (float)zc * 0.125f;
      int n = 0;
#pragma unroll
      for (int q = 0; q < PL; ++q) {
        const bool hv = ev[q] >= lim;
        const uint64_t bal = __ballot(hv);
        const int pos = n + (int)__popcll(bal & lanemask_lt());
        if (hv && pos < kListSlots) {
          st_dev(lw + 1 + 2 * pos, tagged_f32(ev[q], tag));
          st_dev(lw + 2 + 2 * pos, tagged_f32(__uint_as_float((uint32_t)(j0 + lane + kWave * q)), tag));
        }
        n += (int)__popcll(bal);
      }
      if (lane == 0) st_dev(lw, tagged_f32(__uint_as_float((uint32_t)n), tag));
    }
    if (lane == 0) {
      // M_c is the largest of fp32 block maxima, so fp32 holds it exactly
      uint64_t* cs = head_chunk_words(a, head) + 2 * c;
      st_dev(cs, tagged_f32((float)mc, tag));
      st_dev(cs + 1, tagged_f32((float)zc, tag));
      S->flag = atomicAdd(&head_state(a, head)->counter, 1) == nch - 1;
    }
  }
  __syncthreads();
  return S->flag != 0;
}

// The selection of head (b, r), run by the workgroup index_chunk picked: writes the
// ascending selected block ids and their count (and, if asked, one byte per block:
// 1 = selected), and resets the head's arrival counter.  If a word of this call is still
// stale when the bounded wait runs out (or the header asks for that failure), every
// block is selected and the header's status bit and fallback count record it.  Passes
// over blocks or candidates run on all T threads; the chunk statistics, the bin scans,
// the final ranking and the bitmap prefix on wave 0 alone, while the other waves wait at
// the next barrier.  V: the kernel build (select_threshold).
template <int T, int V>
__device__ __forceinline__ void index_select(const IndexArgs& a, int BK, int b, size_t head, IndexSmem<T>* S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.seq_lens[b];
  const int nblk = (N + BK - 1) / BK;
  const int nch = (nblk + a.chunk_blocks - 1) / a.chunk_blocks;
  const int rows = ceil_div(nblk, T);  // block j = row * T + thread
  const uint32_t tag = S->tag;
  TailSmem& sm = S->sm;
  float* s_mass = index_masses<T>(S);
  uint16_t* cand = index_cands<T>(S, rows);
  const uint64_t* e_io = head_block_words(a, head);
  const uint64_t* cs = head_chunk_words(a, head);
  const bool inject = (S->inject & 1) != 0;
  int budget = inject ? 0 : kSpinBudget;
  bool ok = !inject;

  // ---- the head's words, by every thread (one memory round trip): chunk words (M_c, Z_c)
  // into LDS, the first rows of block words into registers
  constexpr int CW = kIdxMaxChunks / T;  // chunk words per thread
  uint64_t x[CW], z[CW];
#pragma unroll
  for (int k = 0; k < CW; ++k) {
    const int i = tid + k * T;
    x[k] = i < nch ? ld_dev(cs + 2 * i) : 0ull;
    z[k] = i < nch ? ld_dev(cs + 2 * i + 1) : 0ull;
  }
  // with lists (index_lists): the chunks' heavy-block lists instead of the first block
  // words, which only the full pass needs (thread tid: chunk tid's count; chunk tid / 8's
  // entry tid % 8)
  static_assert(T >= kListMaxChunks * kListSlots, "one list entry a thread");
  const bool lists = index_lists(a, nblk, nch, T);  // uniform
  uint64_t w[kMassBatch];
#pragma unroll
  for (int u = 0; u < kMassBatch; ++u) {
    const int j = u * T + tid;
    w[u] = (!lists && u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
  }
  const uint64_t* lw = head_list_words(a, head);
  const int lc = tid / kListSlots, ls = tid % kListSlots;
  uint64_t lcw = 0, lvw = 0, liw = 0;
  if (lists) {
    if (tid < nch) lcw = ld_dev(lw + (size_t)tid * kListWords);
    if (lc < nch) {
      lvw = ld_dev(lw + (size_t)lc * kListWords + 1 + 2 * ls);
      liw = ld_dev(lw + (size_t)lc * kListWords + 2 + 2 * ls);
    }
  }
  if (tid < kBins) {
    sm.bmass[tid] = 0;
    sm.bcnt[tid] = 0;
  }
  for (int i = tid; i < kBitWords; i += T) {
    sm.sel[i] = 0;
    sm.tie[i] = 0;
  }
  if (tid == 0) {
    sm.found = 0;
    sm.ncand = 0;
    sm.nfinal = 0;
    sm.ubound = 0u;
    sm.nlist = 0;
    sm.ngath = 0;
    sm.lbad = 0;
    sm.lok = 0;
  }
#pragma unroll
  for (int k = 0; k < CW; ++k) {
    const int i = tid + k * T;
    if (i < nch) {
      S->cm[i] = untag_f32(settle(cs + 2 * i, x[k], tag, budget, ok));
      S->cz[i] = untag_f32(settle(cs + 2 * i + 1, z[k], tag, budget, ok));
    }
  }
  if (lists && tid < nch) {
    sm.lcnt[tid] = (int)__float_as_uint(untag_f32(settle(lw + (size_t)tid * kListWords, lcw, tag, budget, ok)));
    sm.lz[tid] = S->cz[tid];
  }
  // static top-k keeps topk_blocks blocks: the same search with every block weighing 1
  // and P = the number of blocks
  const int kb = a.topk_blocks;
  const bool count = kb > 0;
  const float p = count ? 1.0f : a.top_p[head];
  const bool pick = count ? kb < nblk : (p < 1.0f && nblk > 1);  // else every block is selected
  // Top-p: every block of mass below (1 - p) / (2 nblk) is outside the selection and
  // below its threshold: with total mass ~1 the threshold exceeds (total - p) / nblk.
  // Such blocks stay out of the candidates (peaked heads have thousands of them).
  const uint32_t lbits = count ? 0u : __float_as_uint(fmaxf(0.f, 0.5f * (1.0f - p - 1e-6f) / (float)nblk));
  // first level: 1/8-octave bins (bits >> 20) from the floor up, which span 32 octaves
  // (everything above goes to the top bin); without a floor, half-octave bins from 0
  const int shift1 = lbits ? 20 : 22;
  const uint32_t lo1 = lbits & ~((1u << shift1) - 1u);
  bool failed = __syncthreads_or(!ok) != 0;  // uniform

  // the listed entries this call wrote (slots below their chunk's count), by the threads
  // that hold them; a wait that runs out only rules the lists out here (the full pass
  // below reports it)
  const bool lv = lists && !failed && lc < nch && ls < min(sm.lcnt[lc], kListSlots);
  if (lv) {
    lvw = settle(lw + (size_t)lc * kListWords + 1 + 2 * ls, lvw, tag, budget, ok);
    liw = settle(lw + (size_t)lc * kListWords + 2 + 2 * ls, liw, tag, budget, ok);
    if (!ok) sm.lbad = 1;
  }

  // ---- wave 0: M = max_c M_c (an fp32 value), Z = sum_c Z_c exp(M_c - M); the chunk
  // factors f_c = exp(M_c - M) / Z (fp32) replace the chunk words.  With lists: the
  // number of listed blocks and U, the largest fl(fl(Z_c / 8) f_c) (see below)
  if (!failed && wave == 0) {
    float mloc = -INFINITY;
    for (int i = lane; i < nch; i += kWave) mloc = fmaxf(mloc, S->cm[i]);
    const double M = (double)wave_maxf(mloc);
    double zloc = 0.0;
    for (int i = lane; i < nch; i += kWave) {
      const float cmi = S->cm[i];
      const double e = cmi == -INFINITY ? 0.0 : exp((double)cmi - M);
      zloc += (double)S->cz[i] * e;
      S->cz[i] = (float)e;  // kept until Z is known
    }
    const double invZ = 1.0 / wave_sum(zloc);
    float bl = 0.0f, nl = 0.0f;
    for (int i = lane; i < nch; i += kWave) {
      const float f = (float)((double)S->cz[i] * invZ);
      S->cm[i] = f;
      if (lists) {
        const int n = sm.lcnt[i];
        if (n > kListSlots) sm.lbad = 1;
        nl += (float)n;
        bl = fmaxf(bl, (sm.lz[i] * 0.125f) * f);
      }
    }
    if (lists) {
      bl = wave_maxf(bl);
      nl = wave_sumf(nl);  // at most 256 a chunk over <= 128 chunks: exact in fp32
      if (lane == 0) {
        sm.ubound = __float_as_uint(bl);
        sm.nlist = (int)nl;
      }
    }
  }
  __syncthreads();

  // ---- the lists alone decide when they can.  A block chunk c did not list has e_j <
  // Z_c / 8, so its mass m_j = e_j f_c is at most fl(fl(Z_c / 8) f_c) (rounding is
  // monotone).  With U the largest such bound over the chunks, every block of mass above
  // U is listed; if those blocks reach P in the greedy order (descending key, fixed-point
  // sums as below), every other block ranks after the crossing one, so their prefix is
  // the head's exact selection: their holders gather them, wave 0 ranks them.
  // Otherwise (nothing listed, a list overflowed, a wait ran out, more than kFinal
  // blocks above U, or their mass short of P) the full pass below decides.
  bool decided = false;
  if (lists && pick && !failed && sm.nlist > 0) {  // uniform
    const uint64_t P = (uint64_t)ceil(ldexp((double)p, 62));  // top-p: top-k never uses lists
    const float m = lv ? untag_f32(lvw) * S->cm[lc] : 0.0f;
    const bool g = lv && __float_as_uint(m) > sm.ubound;
    const uint64_t bal = __ballot(g);
    if (bal) {  // uniform
      int base = 0;
      if (lane == 0) base = atomicAdd(&sm.ngath, (int)__popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);
      const int slot = base + (int)__popcll(bal & lanemask_lt());
      if (g && slot < kFinal) {
        sm.fkey[slot] = key_of(m, (int)__float_as_uint(untag_f32(liw)));
        sm.fw[slot] = fixed_bits(__float_as_uint(m));
      }
    }
    __syncthreads();
    if (wave == 0 && !sm.lbad && sm.ngath <= kFinal) {
      const int kept = sm.ngath;
      const bool v = lane < kept;
      const uint64_t my = v ? sm.fkey[lane] : 0ull;
      const uint64_t f = v ? sm.fw[lane] : 0ull;
      uint64_t above = 0;
      for (int i = 0; i < kept; ++i) {
        const uint64_t ki = readlane_u64(my, i), fi = readlane_u64(f, i);
        above += ki > my ? fi : 0ull;
      }
      const uint64_t cb = __ballot(v && above < P && above + f >= P);
      if (cb) {  // every kept block lies above U, the crossing one too
        const uint64_t t = readlane_u64(my, __ffsll((long long)cb) - 1);
        const bool sl = v && my >= t;
        const uint64_t sb = __ballot(sl);
        const int j = (int)(0xFFFFFFFFu - (uint32_t)my);
        int rank = 0;  // selected ids below this one
        for (uint64_t q = sb; q; q &= q - 1) rank += __builtin_amdgcn_readlane(j, __ffsll((long long)q) - 1) < j;
        if (sl) {
          a.sel_idx[head * a.nblk_max + rank] = j;
          atomicOr(&sm.sel[j >> 5], 1u << (j & 31));
        }
        if (lane == 0) {
          sm.total = (int)__popcll(sb);
          sm.lok = 1;
        }
      }
    }
    __syncthreads();
    if (sm.lok) {
      decided = true;
      if (a.sel_mask) {
        uint8_t* m8 = a.sel_mask + head * a.nblk_max;
        for (int j = tid; j < nblk; j += T) m8[j] = (sm.sel[j >> 5] >> (j & 31)) & 1u;
      }
    }
  }

  // ---- every thread: m_j = e_j exp(M_c - M) / Z into LDS; the same pass gathers the
  // candidates (blocks at or above the floor) and builds the first threshold level over
  // them: bin = (bits - lo1) >> shift1, the top bin also takes any larger
  if (!failed && !decided) {
    const int cshift = __ffs(a.chunk_blocks) - 1;
    const float* fch = S->cm;
    for (int i0 = 0; i0 < rows; i0 += kMassBatch) {
      if (i0 > 0 || lists) {
#pragma unroll
        for (int u = 0; u < kMassBatch; ++u) {
          const int j = (i0 + u) * T + tid;
          w[u] = (i0 + u < rows && j < nblk) ? ld_dev(e_io + j) : 0ull;
        }
      }
#pragma unroll
      for (int u = 0; u < kMassBatch; ++u) {
        const int j = (i0 + u) * T + tid;
        if (i0 + u < rows && j < nblk) w[u] = settle(e_io + j, w[u], tag, budget, ok);
      }
#pragma unroll
      for (int u = 0; u < kMassBatch; ++u) {
        if (i0 + u >= rows) break;  // uniform
        const int j = (i0 + u) * T + tid;
        const bool v = j < nblk;
        const float m = v ? untag_f32(w[u]) * fch[j >> cshift] : -1.0f;  // -1: no block
        s_mass[j] = m;
        const uint32_t bits = __float_as_uint(m);
        const bool c = v && pick && bits >= lbits;
        const uint64_t bal = __ballot(c);
        if (bal) {  // uniform
          if (c) {
            const int bin = level_bin(bits, lo1, shift1);
            atomicAdd((unsigned long long*)&sm.bmass[bin], count ? 1ull : (unsigned long long)fixed_bits(bits));
            atomicAdd(&sm.bcnt[bin], 1u);
          }
          int base = 0;
          if (lane == 0) base = atomicAdd(&sm.ncand, (int)__popcll(bal));
          base = __builtin_amdgcn_readfirstlane(base);
          if (c) cand[base + (int)__popcll(bal & lanemask_lt())] = (uint16_t)j;
        }
      }
    }
    failed = __syncthreads_or(!ok) != 0;
  }

  // ---- threshold key: block j is selected iff key_of(m_j, j) >= thr.  A block below the
  // floor is never a candidate and its key lies below every candidate's, so the test
  // holds for every block.
  int* out = a.sel_idx + head * a.nblk_max;
  uint8_t* mask = a.sel_mask ? a.sel_mask + head * a.nblk_max : nullptr;
  const uint64_t P = count ? (uint64_t)kb : (uint64_t)ceil(ldexp((double)p, 62));
  const int ncand = sm.ncand;  // written before the last barrier: uniform
  uint64_t thr = 0;
  bool all = !decided;
  int nsel = decided ? sm.total : 0;  // selected blocks (read by thread 0)
  if (decided) {
  } else if (pick && !failed && ncand <= kFinal) {
    // few candidates (the usual case): wave 0 ranks them exactly, one a lane (the mass of
    // the larger keys decides, as in the last level of the general search), writes the
    // selected ids in ascending order and their count, and leaves the threshold for the
    // mask pass; no crossing (total below p) selects every block
    if (wave == 0) {
      const bool v = lane < ncand;
      const int j = v ? (int)cand[lane] : 0;
      const uint32_t bits = v ? __float_as_uint(s_mass[j]) : 0u;
      const uint64_t my = v ? key_of(__uint_as_float(bits), j) : 0ull;
      const uint64_t f = v ? (count ? 1ull : fixed_bits(bits)) : 0ull;
      uint64_t above = 0;
      for (int i = 0; i < ncand; ++i) {
        const uint64_t ki = readlane_u64(my, i), fi = readlane_u64(f, i);
        above += ki > my ? fi : 0ull;
      }
      const uint64_t cb = __ballot(v && above < P && above + f >= P);
      if (cb) {
        const uint64_t t = readlane_u64(my, __ffsll((long long)cb) - 1);
        const bool sl = v && my >= t;
        const uint64_t sb = __ballot(sl);
        int rank = 0;  // selected ids below this one
        for (uint64_t m = sb; m; m &= m - 1) rank += __builtin_amdgcn_readlane(j, __ffsll((long long)m) - 1) < j;
        if (sl) out[rank] = j;
        if (lane == 0) {
          sm.thr = t;
          sm.found = 1;
          sm.total = (int)__popcll(sb);
        }
      }
    }
    __syncthreads();
    if (sm.found) {
      all = false;
      thr = uni64(sm.thr);
      nsel = sm.total;
      if (mask)
        for (int j = tid; j < nblk; j += T) mask[j] = key_of(s_mass[j], j) >= thr;
    }
  } else if (pick && !failed) {
    if (wave == 0) {
      scan_level(0, P, lo1, 0xFFFFFFFFu, shift1, sm);
      // the pruned blocks were not counted: the candidates start at the floor
      if (lane == 0 && sm.found) sm.lo = min(max(sm.lo, lbits), sm.hi);
    }
    __syncthreads();
    if (sm.found) {  // else the total mass is below p: every block
      all = false;
      thr = select_threshold<T, V>(s_mass, cand, ncand, nblk, P, sm, count);
      // ordered compaction of the selected ids (ascending): one ballot per unit of 64
      // blocks (row i, wave w: blocks i T + 64 w ..) into a bitmap, no atomics; then every
      // wave scans the units' counts itself (lane l holds units 4 l .. 4 l + 3) and writes
      // its own units' ids at their ranks, so no further barrier is needed
      constexpr int W = T / kWave;
      for (int i = 0; i < rows; ++i) {
        const int j = i * T + tid;
        const uint64_t bal = __ballot(j < nblk && key_of(s_mass[j], j) >= thr);
        const int w0 = 2 * (i * W + wave);
        if (lane == 0) sm.sel[w0] = (uint32_t)bal;
        if (lane == 32) sm.sel[w0 + 1] = (uint32_t)(bal >> 32);
      }
      __syncthreads();
      static_assert(4 * kWave * 2 >= kBitWords, "a wave's lanes cover every unit");
      const int nunits = rows * W;
      uint32_t uc[4], v = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int u = 4 * lane + k;
        uc[k] = u < nunits ? (uint32_t)(__popc(sm.sel[2 * u]) + __popc(sm.sel[2 * u + 1])) : 0u;
        v += uc[k];
      }
      const uint32_t incl = wave_incl_scan_u32(v);
      const uint32_t excl = incl - v;
      nsel = (int)__builtin_amdgcn_readlane(incl, 63);
      for (int i = 0; i < rows; ++i) {
        const int u = i * W + wave, ul = u >> 2, uk = u & 3;  // held by lane ul, slot uk
        const uint32_t pre = __builtin_amdgcn_readlane(excl, ul) +
                             (uk > 0 ? __builtin_amdgcn_readlane(uc[0], ul) : 0u) +
                             (uk > 1 ? __builtin_amdgcn_readlane(uc[1], ul) : 0u) +
                             (uk > 2 ? __builtin_amdgcn_readlane(uc[2], ul) : 0u);
        const uint64_t bal = ((uint64_t)sm.sel[2 * u + 1] << 32) | sm.sel[2 * u];
        const int j = i * T + tid;
        const bool sl = (bal >> lane) & 1ull;
        if (sl) out[pre + (uint32_t)__popcll(bal & lanemask_lt())] = j;
        if (mask && j < nblk) mask[j] = sl;
      }
    }
  }
  if (all) {
    select_all<T>(a, head, nblk);
    if (failed && tid == 0) {
      atomicOr(&a.hdr->status, (uint32_t)RTP_INDEX_WAIT_EXPIRED);
      atomicAdd(&a.hdr->fallbacks, 1u);
    }
  }
  if (tid == 0) {
    if (!all) a.sel_cnt[head] = nsel;
    __hip_atomic_store(&head_state(a, head)->counter, 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
  }
}

// After the selection: the head's tag advances for the next call.  When it wraps (after
// 2^32 - 1 calls), the head's words are cleared first, so no word written under an old
// tag can carry a new one.
template <int T>
__device__ __forceinline__ void index_advance_tag(const IndexArgs& a, size_t head, uint32_t tag) {
  const uint32_t nt = next_tag(tag);
  if (nt == 1u) {
    uint64_t* w = head_chunk_words(a, head);
    const int n = 2 * a.n_chunk_cap + a.nblk_max + index_list_cap(a.nblk_max) * kListWords;
    for (int i = threadIdx.x; i < n; i += T) st_dev(w + i, 0ull);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&head_state(a, head)->tag, nt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace rtp
