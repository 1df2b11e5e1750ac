// Device code of kernel 2 (block-sparse split attention over the index kernel's
// selection) and of the local heads' window + sink attention.
//
// Kernel 2: exact softmax(q K^T / sqrt(128)) V over only the blocks the index kernel
// selected, split along the context ("Full Attention Strikes Back", method item 2 and
// architecture paragraph: Kernel 2 at D128 with a cross-split reduce).  Workgroup =
// (split, KV group, sequence); it builds the union of its retrieval heads' selected
// blocks inside the split (binary search into each ascending list, LDS head-mask per
// block, ordered compaction), so a block picked by several heads of the group is read
// from HBM once (with the index kernel's per-head block masks the union is one round of
// byte loads), then streams the union's 16-token sub-tiles through the shared
// attention core (rtp_attn.hpp) and emits per-head (o, lse) partials.
//
// Local heads: the same core over attention sinks + the sliding window (RTPurbo
// review, Adaptive sparse attention: local heads keep only window + sinks).
// Workgroup = (split, KV group, sequence); split 0 holds the sinks, splits 1.. hold
// consecutive window chunks.
#pragma once

#include "rtp_attn.hpp"

namespace rtp {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kMaxSplitBlocks = 2048;
constexpr int kOrderMax = 256;  // KV groups (sequences x KV heads) kernel 2 orders by weight

template <int G>
struct SparseSmem {
  uint32_t hm[kMaxSplitBlocks / 4];  // per block of the split: head mask, one byte each
  uint32_t list[kMaxSplitBlocks];    // the union in ascending order: (offset << 8) | mask
  int wcnt[kAttnWaves];
  float m[kAttnWaves * G], l[kAttnWaves * G];
  float acc[kAttnWaves * G * kHeadDim];
  int gw[kOrderMax];  // per KV group: selected blocks summed over its retrieval heads
  int pick;
};
template <int G>
struct LocalSmem {
  float m[kAttnWaves * G], l[kAttnWaves * G];
  float acc[kAttnWaves * G * kHeadDim];
};

// Window split of the local heads: >= ~1024 workgroups over the batch, 64..4096 tokens a
// split; split 0 holds the sinks, so there are 1 + ceil(window / split) splits.
inline int local_split_tokens(int B, int Hkv, int window) {
  const long long groups = (long long)B * Hkv;
  int st = 4096;
  while (st > 64 && groups * ceil_div(window > 1 ? window : 1, st) < 1024) st >>= 1;
  return st;
}

struct SparseArgs {
  const uint16_t *q, *kc, *vc;  // bf16 [B, Hq, 128], [B, Hkv, max_ctx, 128] x2
  const int* seq_lens;
  const int* ret_heads;
  const int* sel_idx;
  const int* sel_cnt;
  const uint8_t* sel_mask;  // [B, n_ret, nblk_max] 1 = selected, or null (then the lists)
  int Hq, Hkv, n_ret, max_ctx, nblk_max, split_blocks;
};
struct LocalArgs {
  const uint16_t *q, *kc, *vc;
  const int* seq_lens;
  const int* loc_heads;
  int Hq, Hkv, n_loc, max_ctx, window, sinks, split_tokens;
};

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

// Kernel 2's dispatch order of KV groups: the group of rank `rank` when groups are taken
// heaviest first (most selected blocks summed over their retrieval heads, ties by
// index), so the grid ends with its lightest workgroups and drains quickly.  Returns
// b * Hkv + g.  Without the counts (block masks only) or with more than kOrderMax
// groups, the natural order.  Every thread of the workgroup calls it.
template <int G>
__device__ __forceinline__ int group_of_rank(const SparseArgs& a, int B, int rank, SparseSmem<G>* S) {
  const int ngrp = B * a.Hkv;
  if (!a.sel_cnt || ngrp > kOrderMax) return rank;
  const int tid = threadIdx.x;
  for (int k = tid; k < ngrp; k += kAttnThreads) S->gw[k] = 0;
  __syncthreads();
  for (int i = tid; i < B * a.n_ret; i += kAttnThreads) {
    const int b = i / a.n_ret, r = i - b * a.n_ret;
    atomicAdd(&S->gw[b * a.Hkv + a.ret_heads[r] / G], a.sel_cnt[i]);
  }
  __syncthreads();
  for (int k = tid; k < ngrp; k += kAttnThreads) {
    const int wk = S->gw[k];
    int rk = 0;
    for (int k2 = 0; k2 < ngrp; ++k2) {
      const int w2 = S->gw[k2];
      rk += (w2 > wk) || (w2 == wk && k2 < k);
    }
    if (rk == rank) S->pick = k;
  }
  __syncthreads();
  return S->pick;
}

// Split c of KV group g of sequence b.  emit(i, d, o, lse) takes retrieval head i's dim d
// (lse once, at d == 0); a split past the sequence's end emits o = 0, lse = -inf.  A
// group without retrieval heads emits nothing and returns false.
template <int BK, int G, class Emit>
__device__ __forceinline__ bool sparse_split(const SparseArgs& a, int c, int g, int b, SparseSmem<G>* S,
                                             Emit emit) {
  constexpr int ST = BK / 16;  // sub-tiles per block
  constexpr int kWaves = kAttnWaves, kThreads = kAttnThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_ret = a.n_ret, Hq = a.Hq, nblk_max = a.nblk_max, split_blocks = a.split_blocks;
  const int* __restrict__ ret_heads = a.ret_heads;
  const int* __restrict__ sel_idx = a.sel_idx;
  const int* __restrict__ sel_cnt = a.sel_cnt;
  const uint8_t* __restrict__ sel_mask = a.sel_mask;
  // the sequence length and (for the lists) the first 64 selected counts go out with the
  // head list: one memory round trip
  const int N = a.seq_lens[b];
  const int cnt_l = (!sel_mask && lane < n_ret) ? sel_cnt[(size_t)b * n_ret + lane] : 0;
  int rbeg, rend;
  group_range(ret_heads, n_ret, g, G, rbeg, rend);
  const int nh = rend - rbeg;
  if (nh == 0) return false;
  const int nblk = (N + BK - 1) / BK;
  const int jlo = c * split_blocks, jhi = min(jlo + split_blocks, nblk);
  uint32_t* s_hm = S->hm;
  uint32_t* s_list = S->list;
  int* s_wcnt = S->wcnt;

  int nL = 0;
  if (jlo < jhi) {
    const int nb = jhi - jlo;
    // per block of the split, the mask of the group's heads that selected it (one byte
    // per block in s_hm); each wave then takes a contiguous segment of blocks
    const int seg = ((nb + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int sb = wave * seg, se = min(nb, sb + seg);
    uint8_t* hm8 = reinterpret_cast<uint8_t*>(s_hm);
    int cnt = 0;
    if (sel_mask) {
      // block masks: each lane ORs the group's heads' bytes of its blocks (one round trip)
      const uint8_t* mrow = sel_mask + ((size_t)b * n_ret + rbeg) * nblk_max + jlo;
      for (int base = sb; base < se; base += 64) {
        const int off = base + lane;
        uint32_t mk = 0;
        if (off < se) {
#pragma unroll
          for (int h = 0; h < G; ++h)
            if (h < nh && mrow[(size_t)h * nblk_max + off]) mk |= 1u << h;
          hm8[off] = (uint8_t)mk;
        }
        cnt += __popcll(__ballot(mk != 0));
      }
    } else {
      for (int i = tid; i < (nb + 3) / 4; i += kThreads) s_hm[i] = 0;
      __syncthreads();
      // mark each head's selected blocks in [jlo, jhi): one wave per head.  A list of at
      // most 64 entries is read in one round; a longer one is searched for its range.
      for (int h = wave; h < nh; h += kWaves) {
        const int hh = rbeg + h;
        const size_t hr = (size_t)b * n_ret + hh;
        const int cnt_h = hh < 64 ? __shfl(cnt_l, hh) : sel_cnt[hr];
        const int* sl = sel_idx + hr * nblk_max;
        const uint32_t bit = 1u << h;
        if (cnt_h <= 64) {
          const int v = lane < cnt_h ? sl[lane] : -1;
          if (v >= jlo && v < jhi) atomicOr(&s_hm[(v - jlo) >> 2], bit << (((v - jlo) & 3) * 8));
        } else {
          const int a0 = lower_bound_wave(sl, cnt_h, jlo);
          const int e0 = lower_bound_wave(sl, cnt_h, jhi);
          for (int i = a0 + lane; i < e0; i += 64) {
            const int off = sl[i] - jlo;
            atomicOr(&s_hm[off >> 2], bit << ((off & 3) * 8));
          }
        }
      }
      __syncthreads();
      for (int base = sb; base < se; base += 64) {
        const int off = base + lane;
        const uint32_t mk = off < se ? hm8[off] : 0u;
        cnt += __popcll(__ballot(mk != 0));
      }
    }
    // ordered compaction of the blocks some head selected: entry = (offset << 8) | mask
    if (lane == 0) s_wcnt[wave] = cnt;
    __syncthreads();
    int pos = 0;
    for (int w = 0; w < wave; ++w) pos += s_wcnt[w];
    for (int base = sb; base < se; base += 64) {
      const int off = base + lane;
      const uint32_t mk = off < se ? hm8[off] : 0u;
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
    qk[h] = h < nh ? ld16(a.q + ((size_t)b * Hq + ret_heads[rbeg + h]) * kHeadDim + c16 * 8)
                   : make_uint4(0, 0, 0, 0);
  const size_t kvoff = ((size_t)b * a.Hkv + g) * (size_t)a.max_ctx * kHeadDim;
  const float scale = (float)(kLog2e / 11.313708498984761);  // log2(e) / sqrt(128)
  auto item = [&](int i, int& row0, uint32_t& hm) {
    const uint32_t ent = s_list[i / ST];
    row0 = (jlo + (int)(ent >> 8)) * BK + 16 * (i % ST);
    hm = row0 < N ? (ent & 0xffu) : 0u;
  };
  attn_stream<G, kWaves>(st, a.kc + kvoff, a.vc + kvoff, nL * ST, N, item, qk, scale, wave, lane);
  attn_publish_wave<G, kWaves>(st, S->m, S->l, S->acc, wave, lane);
  __syncthreads();
  for (int idx = tid; idx < nh * kHeadDim; idx += kThreads) {
    const int h = idx >> 7, d = idx & (kHeadDim - 1);
    float o, lse;
    attn_merge<G, kWaves>(S->m, S->l, S->acc, h, d, o, lse);
    emit(rbeg + h, d, o, lse);
  }
  return true;
}

// Split c of the local heads of KV group g of sequence b; emit(i, d, o, lse) takes local
// head i's dim d (lse once, at d == 0), also for an empty split (o = 0, lse = -inf).
// Returns false, emitting nothing, for a group without local heads.
template <int G, class Emit>
__device__ __forceinline__ bool local_split(const LocalArgs& a, int c, int g, int b, LocalSmem<G>* S,
                                            Emit emit) {
  constexpr int kWaves = kAttnWaves, kThreads = kAttnThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int* __restrict__ loc_heads = a.loc_heads;
  const int sinks = a.sinks, window = a.window, split_tokens = a.split_tokens;
  int ibeg, iend;
  group_range(loc_heads, a.n_loc, g, G, ibeg, iend);
  const int nh = iend - ibeg;
  if (nh == 0) return false;
  const int N = a.seq_lens[b];
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

  AttnState<G> st;
  attn_init(st);
  uint4 qk[G];
  const int c16 = lane & 15;
#pragma unroll
  for (int h = 0; h < G; ++h)
    qk[h] = h < nh ? ld16(a.q + ((size_t)b * a.Hq + loc_heads[ibeg + h]) * kHeadDim + c16 * 8)
                   : make_uint4(0, 0, 0, 0);
  const size_t kvoff = ((size_t)b * a.Hkv + g) * (size_t)a.max_ctx * kHeadDim;
  const float scale = (float)(kLog2e / 11.313708498984761);
  const uint32_t allh = (1u << nh) - 1u;
  auto item = [&](int i, int& row0, uint32_t& hm) {
    row0 = t0 + 16 * i;
    hm = allh;
  };
  attn_stream<G, kWaves>(st, a.kc + kvoff, a.vc + kvoff, nitems, t1, item, qk, scale, wave, lane);
  attn_publish_wave<G, kWaves>(st, S->m, S->l, S->acc, wave, lane);
  __syncthreads();
  for (int idx = tid; idx < nh * kHeadDim; idx += kThreads) {
    const int h = idx >> 7, d = idx & (kHeadDim - 1);
    float o, lse;
    attn_merge<G, kWaves>(S->m, S->l, S->acc, h, d, o, lse);
    emit(ibeg + h, d, o, lse);
  }
  return true;
}

}  // namespace rtp
