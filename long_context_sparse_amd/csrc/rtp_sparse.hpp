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
  // kernel 2's ordering of KV groups: per group, selected blocks summed over its
  // retrieval heads and its number of retrieval heads; the head list; the lengths
  int gw[kOrderMax], gn[kOrderMax], rh[kOrderMax], sl[kOrderMax], slot[kOrderMax];
  int pick;
};
template <int G>
struct LocalSmem {
  float m[kAttnWaves * G], l[kAttnWaves * G];
  float acc[kAttnWaves * G * kHeadDim];
};

// Window split of the local heads: >= ~1024 workgroups over the batch where splits of at
// least 128 tokens allow (a shorter split leaves each wave one 16-token sub-tile and the
// merge more partials than it saves), 128..4096 tokens a split; split 0 holds the sinks,
// so there are 1 + ceil(window / split) splits.
inline int local_split_tokens(int B, int Hkv, int window) {
  const long long groups = (long long)B * Hkv;
  int st = 4096;
  while (st > 128 && groups * ceil_div(window > 1 ? window : 1, st) < 1024) st >>= 1;
  return st;
}

struct SparseArgs {
  const uint16_t *q, *kc, *vc;  // bf16 [B, Hq, 128], [B, Hkv, max_ctx, 128] x2
  const int* seq_lens;
  const int* ret_heads;
  const int* sel_idx;
  const int* sel_cnt;
  const uint8_t* sel_mask;  // [B, n_ret, nblk_max] 1 = selected, or null (then the lists)
  const int* kv_slot;       // [Hkv] KV group -> its index in the caches (>= 0), or null (identity)
  int Hq, Hkv, n_ret, max_ctx, nblk_max, split_blocks;
  int n_full;               // groups in the caches (Hkv when kv_slot is null)
};
struct LocalArgs {
  const uint16_t *q, *kc, *vc;
  const int* seq_lens;
  const int* loc_heads;
  int Hq, Hkv, n_loc, max_ctx, window, sinks, split_tokens;
  // KV placement: kv_slot[g] >= 0: group g's rows are in kc/vc at group index kv_slot[g]
  // ([B, n_full, max_ctx, 128]); < 0: in the sink + window ring kr/vr at group index
  // -1 - kv_slot[g] ([B, n_ring, sinks + window, 128]).  Null: identity, all in kc/vc.
  const int* kv_slot;
  const uint16_t *kr, *vr;
  int n_full, n_ring;
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

// Kernel 2's workgroup: sequence b, KV group g, the range [rbeg, rbeg + nh) of the
// ascending retrieval-head list that falls in g, their query-head ids (hid[h] for h >=
// nh repeats the last one, so loads through it stay valid) and the sequence length.
template <int G>
struct SparseGroup {
  int b, g, N, rbeg, nh, slot;
  int hid[G];
};

// Kernel 2's dispatch order of KV groups: the group of rank `rank` when groups are taken
// heaviest first (most selected blocks summed over their retrieval heads, ties by
// index), so the grid ends with its lightest workgroups and drains quickly.  The
// selected counts, the head list and the lengths come in one round of loads, so the
// group's heads and length are known without a further round trip.  Without the counts
// (block masks only), or with more than kOrderMax groups or retrieval heads, the natural
// order.  Every thread of the workgroup calls it.
template <int G>
__device__ __forceinline__ SparseGroup<G> sparse_group(const SparseArgs& a, int B, int rank, SparseSmem<G>* S) {
  const int Hkv = a.Hkv, n_ret = a.n_ret;
  const int ngrp = B * Hkv;
  const int tid = threadIdx.x;
  SparseGroup<G> r;
  int beg, nh;
  if (a.sel_cnt && ngrp <= kOrderMax && n_ret <= kOrderMax) {
    // the first (head, count) of every thread and the lengths: unconditional loads at
    // clamped indices, all in flight while the tables are cleared
    const int nbr = B * n_ret;
    const int i0 = min(tid, nbr - 1), b0 = i0 / n_ret, r0 = i0 - b0 * n_ret;
    const int h0 = a.ret_heads[r0], c0 = a.sel_cnt[i0];
    const int len0 = a.seq_lens[min(tid, B - 1)];  // B <= kOrderMax == kAttnThreads
    const int* slot_src = a.kv_slot ? a.kv_slot : a.seq_lens;  // any readable word without a table
    const int slot0 = slot_src[a.kv_slot ? min(tid, Hkv - 1) : 0];
    for (int k = tid; k < ngrp; k += kAttnThreads) S->gw[k] = 0;
    for (int k = tid; k < Hkv; k += kAttnThreads) S->gn[k] = 0;
    __syncthreads();
    if (tid < B) S->sl[tid] = len0;
    if (tid < Hkv) S->slot[tid] = a.kv_slot ? slot0 : tid;
    auto add = [&](int b, int rr, int h, int cnt) {
      if (h >= 0 && h < a.Hq) {
        atomicAdd(&S->gw[b * Hkv + h / G], cnt);
        if (b == 0) atomicAdd(&S->gn[h / G], 1);
      }
      if (b == 0) S->rh[rr] = h;
    };
    if (tid < nbr) add(b0, r0, h0, c0);
    for (int i = tid + kAttnThreads; i < nbr; i += kAttnThreads) {
      const int b = i / n_ret, rr = i - b * n_ret;
      add(b, rr, a.ret_heads[rr], a.sel_cnt[i]);
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
    const int k = S->pick;
    r.b = k / Hkv;
    r.g = k - r.b * Hkv;
    beg = 0;
    for (int g2 = 0; g2 < r.g; ++g2) beg += S->gn[g2];
    nh = S->gn[r.g];
    r.N = S->sl[r.b];
    r.slot = S->slot[r.g];
#pragma unroll
    for (int h = 0; h < G; ++h) r.hid[h] = nh > 0 ? S->rh[beg + min(h, nh - 1)] : 0;
  } else {
    r.b = rank / Hkv;
    r.g = rank - r.b * Hkv;
    r.N = a.seq_lens[r.b];
    r.slot = a.kv_slot ? a.kv_slot[r.g] : r.g;
    int end;
    group_range(a.ret_heads, n_ret, r.g, G, beg, end);
    nh = end - beg;
#pragma unroll
    for (int h = 0; h < G; ++h) r.hid[h] = nh > 0 ? a.ret_heads[beg + min(h, nh - 1)] : 0;
  }
  r.rbeg = beg;
  r.nh = nh;
  return r;
}

// Split c of the workgroup's KV group (sparse_group).  emit(i, d, o, lse) takes retrieval
// head i's dim d (lse once, at d == 0); a split past the sequence's end emits o = 0,
// lse = -inf.  A group without retrieval heads emits nothing and returns false.
template <int BK, int G, class Emit>
__device__ __forceinline__ bool sparse_split(const SparseArgs& a, int c, const SparseGroup<G>& grp,
                                             SparseSmem<G>* S, Emit emit) {
  constexpr int ST = BK / 16;  // sub-tiles per block
  constexpr int kWaves = kAttnWaves, kThreads = kAttnThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_ret = a.n_ret, Hq = a.Hq, nblk_max = a.nblk_max, split_blocks = a.split_blocks;
  const int* __restrict__ sel_idx = a.sel_idx;
  const int* __restrict__ sel_cnt = a.sel_cnt;
  const uint8_t* __restrict__ sel_mask = a.sel_mask;
  const int b = grp.b, g = grp.g, N = grp.N, rbeg = grp.rbeg, nh = grp.nh;
  if (nh == 0) return false;
  // the query rows go out first (unconditional loads: a head slot past nh reads the last
  // head's row), in flight while the split's blocks are gathered
  uint4 qk[G];
  const int c16 = lane & 15;
#pragma unroll
  for (int h = 0; h < G; ++h) qk[h] = ld16(a.q + ((size_t)b * Hq + grp.hid[h]) * kHeadDim + c16 * 8);
  const int cnt_l = (!sel_mask && lane < n_ret) ? sel_cnt[(size_t)b * n_ret + lane] : 0;
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
      // block masks: each lane ORs the group's heads' bytes of its blocks.  The loads are
      // unconditional (clamped to the last head and block), so all G are in flight at once.
      const uint8_t* mrow = sel_mask + ((size_t)b * n_ret + rbeg) * nblk_max + jlo;
      for (int base = sb; base < se; base += 64) {
        const int off = base + lane;
        const int offc = min(off, se - 1);
        uint32_t v[G];
#pragma unroll
        for (int h = 0; h < G; ++h) v[h] = mrow[(size_t)min(h, nh - 1) * nblk_max + offc];
        uint32_t mk = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) mk |= (h < nh && v[h] != 0u) ? 1u << h : 0u;
        if (off >= se) mk = 0;
        if (off < se) hm8[off] = (uint8_t)mk;
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
  // a group whose rows are not in the full caches (a caller error: it has retrieval
  // heads) reads nothing and emits empty partials
  if (grp.slot < 0) nL = 0;
  const size_t kvoff = ((size_t)b * a.n_full + max(grp.slot, 0)) * (size_t)a.max_ctx * kHeadDim;
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
  const int slot = a.kv_slot ? a.kv_slot[g] : g;
  const int s_end = min(sinks, N);
  // the window's rows: positions [max(s_end, N - window), N) of the full cache, or every
  // stored ring row past the sinks: the ring holds positions < sinks at their own row and
  // the last `window` positions at rows sinks + (p - sinks) mod window, so its rows
  // [s_end, min(N, sinks + window)) are exactly the window (in another order)
  const bool ring = slot < 0;
  const int w0 = ring ? s_end : max(s_end, N - window);
  const int w1 = ring ? min(N, sinks + window) : N;
  int t0, t1;
  if (c == 0) {
    t0 = 0;
    t1 = s_end;
  } else {
    t0 = w0 + (c - 1) * split_tokens;
    t1 = min(w1, t0 + split_tokens);
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
  const size_t kvoff = ring ? ((size_t)b * a.n_ring + (-1 - slot)) * (size_t)(sinks + window) * kHeadDim
                            : ((size_t)b * a.n_full + slot) * (size_t)a.max_ctx * kHeadDim;
  const uint16_t* kbase = ring ? a.kr : a.kc;
  const uint16_t* vbase = ring ? a.vr : a.vc;
  const float scale = (float)(kLog2e / 11.313708498984761);
  const uint32_t allh = (1u << nh) - 1u;
  auto item = [&](int i, int& row0, uint32_t& hm) {
    row0 = t0 + 16 * i;
    hm = allh;
  };
  attn_stream<G, kWaves>(st, kbase + kvoff, vbase + kvoff, nitems, t1, item, qk, scale, wave, lane);
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

// The local heads' partials in a workspace: lse [B, n_loc, n_split], then o [B, n_loc,
// n_split, 128], for a window split of split_tokens (split 0 holds the sinks).
struct LocalLayout {
  int split_tokens, n_split;
  size_t off_lse, off_o, total;
};
inline LocalLayout local_layout_for(int B, int n_loc, int window, int split_tokens) {
  LocalLayout L{};
  L.split_tokens = split_tokens;
  L.n_split = 1 + ceil_div(window, split_tokens);
  L.off_lse = 0;
  L.off_o = align_up((size_t)B * n_loc * L.n_split * sizeof(float), 256);
  L.total = L.off_o + align_up((size_t)B * n_loc * L.n_split * kHeadDim * sizeof(float), 256);
  return L;
}
// Host checks of the local heads' arguments shared by rtp_local_window_attn and the
// decode step's attention launch (n_loc > 0); fills L with `layout`'s split.
template <class LayoutFn>
inline rtp_status local_args_check(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                                   const int* loc_heads, int B, int Hq, int Hkv, int n_loc, int max_ctx, int window,
                                   int sinks, const void* workspace, size_t ws_bytes, const int* kv_slot, int n_full,
                                   const void* k_ring, const void* v_ring, int n_ring, LayoutFn layout,
                                   LocalLayout& L) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_loc < 0 || n_loc > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv || window < 0 || sinks < 0 || window + sinks < 1) return RTP_EINVAL;
  {
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return RTP_EUNSUPPORTED;
  }
  if (!q || !seq_lens || !loc_heads || !workspace) return RTP_EINVAL;
  if (kv_slot) {
    // full caches may be absent when every group is in the ring, and the reverse
    if (n_full < 0 || n_full > Hkv || n_ring < 0 || n_ring > Hkv || n_full + n_ring < 1 || n_full + n_ring > Hkv)
      return RTP_EINVAL;
    if (n_full > 0 && (!k_cache || !v_cache)) return RTP_EINVAL;
    if (n_ring > 0 && (!k_ring || !v_ring)) return RTP_EINVAL;
    if (((uintptr_t)k_ring | (uintptr_t)v_ring) & 15) return RTP_EINVAL;
  } else if (!k_cache || !v_cache) {
    return RTP_EINVAL;
  }
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return RTP_EINVAL;
  if ((uintptr_t)workspace & 255) return RTP_EINVAL;
  L = layout(B, Hkv, n_loc, window < max_ctx ? window : max_ctx);
  if (ws_bytes < L.total) return RTP_EINVAL;
  if (L.n_split > 65535 || B > 65535) return RTP_EUNSUPPORTED;
  return RTP_OK;
}

// the local heads' window split (256-thread workgroups)
inline LocalLayout local_layout(int B, int Hkv, int n_loc, int window) {
  return local_layout_for(B, n_loc, window, local_split_tokens(B, Hkv, window));
}

}  // namespace rtp
