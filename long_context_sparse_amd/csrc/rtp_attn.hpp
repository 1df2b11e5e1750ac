// Decode attention core shared by the block-sparse split kernel and the local
// window kernel: one wave64 streams 16-token sub-tiles of one KV head's K and V
// (bf16, head_dim 128) and keeps an online softmax for up to G query heads of the
// KV group, so every K/V byte is read once for all heads that need it.
//
// Lane layout of a 16-token sub-tile (4 KB of K, 4 KB of V): one 16-byte load per
// lane covers 4 consecutive rows (1 KB contiguous); lane l holds dims
// 8*(l & 15) .. +8 of rows 4*i + (l >> 4), i = 0..3.  A query-key dot product is a
// packed bf16 dot (v_dot2) per dword, then a 16-lane transpose-reduce leaves lane l
// with the full logit of row 4*((l >> 2) & 3) + (l >> 4) (4 replicas).  Softmax
// statistics are kept in the base-2 domain.  Every cross-lane step is a DPP lane move
// inside a 16-lane row, so the inner loop issues no LDS traffic.
#pragma once

#include "rtp_common.hpp"

namespace rtp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int G>
struct AttnState {
  float m[G];       // running max (log2 domain), wave-uniform
  float l[G];       // per-lane partial denominators (one replica of each row counted)
  float acc[G][8];  // per-lane partial numerators for this lane's 8 dims
};

template <int G>
__device__ __forceinline__ void attn_init(AttnState<G>& s) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    s.m[h] = -INFINITY;
    s.l[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s.acc[h][k] = 0.f;
  }
}

struct SubTile {
  uint4 k[4], v[4];
};

// Loads rows [row0, row0 + 16) of kg/vg (row stride 128) with streaming loads (each K/V
// byte is read once).  A row at or beyond row_end reads row min(row, row_end - 1)
// instead (row 0 when row_end <= 0), so every load is unconditional and in bounds;
// attn_subtile masks those rows.  Branch-free loads let the compiler count them, so the
// next sub-tile's loads stay in flight while the current one is computed.
__device__ __forceinline__ void load_subtile(SubTile& t, const uint16_t* __restrict__ kg,
                                             const uint16_t* __restrict__ vg, int row0, int row_end,
                                             int lane) {
  const int R = lane >> 4, c16 = lane & 15;
  const int last = max(row_end - 1, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = min(row0 + 4 * i + R, last);
    const size_t off = (size_t)row * kHeadDim + c16 * 8;
    t.k[i] = ld16_nt(kg + off);
    t.v[i] = ld16_nt(vg + off);
  }
}

// Online-softmax update with one loaded sub-tile.  Rows at or beyond row_end are
// masked (their logits are -inf and their V rows zero, whatever was loaded for them);
// hmask picks the heads (bit h) that attend to these rows and must be 0 unless
// row0 < row_end.  qk[h] holds head h's 8 query dims of this lane.
//
// The running maximum changes only when a logit exceeds it (a wave-wide ballot); most
// sub-tiles then skip the maximum reduction and the rescaling of the accumulators, with
// the same result as the unconditional update (their rescale factor would be exactly 1).
template <int G>
__device__ __forceinline__ void attn_subtile(AttnState<G>& s, const SubTile& tile, int row0,
                                             int row_end, uint32_t hmask, const uint4 (&qk)[G],
                                             float scale_log2, int lane) {
  const int R = lane >> 4;
  const int isel = (lane >> 2) & 3;
  const bool myvalid = row0 + 4 * isel + R < row_end;
  const bool b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
  const bool counted = (lane & 3) == 0;
  // V rows in fp32, unpacked once for all heads; rows past row_end are zero
  float vf[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = tile.v[i];
    vf[i][0] = bf_lo(v.x);
    vf[i][1] = bf_hi(v.x);
    vf[i][2] = bf_lo(v.y);
    vf[i][3] = bf_hi(v.y);
    vf[i][4] = bf_lo(v.z);
    vf[i][5] = bf_hi(v.z);
    vf[i][6] = bf_lo(v.w);
    vf[i][7] = bf_hi(v.w);
  }
  if (row0 + 16 > row_end) {  // wave-uniform: only a sequence's last sub-tile is ragged
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = row0 + 4 * i + R < row_end;
#pragma unroll
      for (int k = 0; k < 8; ++k) vf[i][k] = ok ? vf[i][k] : 0.f;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!((hmask >> h) & 1u)) continue;
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = dot2(tile.k[i].x, qk[h].x, 0.f);
      a = dot2(tile.k[i].y, qk[h].y, a);
      a = dot2(tile.k[i].z, qk[h].z, a);
      part[i] = dot2(tile.k[i].w, qk[h].w, a);
    }
    // transpose-reduce over the 16 lanes that share R (one DPP row), on DPP lane moves:
    // the row mirror (partner l ^ 15) exchanges parts by bit 3, the half-row mirror
    // (partner l ^ 7) by bit 2, then xor 2 and xor 1 finish the row sum
    const float x0 = b3 ? part[0] : part[2];
    const float x1 = b3 ? part[1] : part[3];
    const float y0 = dpp_f32<kDppMirror>(x0);
    const float y1 = dpp_f32<kDppMirror>(x1);
    const float k0 = (b3 ? part[2] : part[0]) + y0;
    const float k1 = (b3 ? part[3] : part[1]) + y1;
    const float xs = b2 ? k0 : k1;
    float v = (b2 ? k1 : k0) + dpp_f32<kDppHalfMirror>(xs);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppXor1>(v);
    const float lg = myvalid ? v * scale_log2 : -INFINITY;
    if (__ballot(lg > s.m[h]) != 0ull) {
      const float mnew = fmaxf(s.m[h], wave_maxf(lg));
      const float alpha = fast_exp2(s.m[h] - mnew);
      s.l[h] *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) s.acc[h][k] *= alpha;
      s.m[h] = mnew;
    }
    const float p = fast_exp2(lg - s.m[h]);
    s.l[h] += counted ? p : 0.f;
    // p of row 4 * i + R sits in lane 4 * i of this lane's DPP row
    float pi[4];
    pi[0] = dpp_f32<kDppRowBcast0>(p);
    pi[1] = dpp_f32<kDppRowBcast0 + 4>(p);
    pi[2] = dpp_f32<kDppRowBcast0 + 8>(p);
    pi[3] = dpp_f32<kDppRowBcast0 + 12>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) s.acc[h][k] = fmaf(pi[i], vf[i][k], s.acc[h][k]);
  }
}

// Streams this wave's items i = wave, wave + WAVES, ... through attn_subtile with the
// next item's loads in flight while the current one is computed (two sub-tile buffers
// used in turn, so no registers are copied).  item(i, row0, hmask) gives the first row
// and the head mask of item i (hmask 0 skips it).
template <int G, int WAVES, class ItemFn>
__device__ __forceinline__ void attn_stream(AttnState<G>& s, const uint16_t* __restrict__ kg,
                                            const uint16_t* __restrict__ vg, int nitems, int row_end,
                                            ItemFn item, const uint4 (&qk)[G], float scale_log2,
                                            int wave, int lane) {
  int i = wave;
  if (i >= nitems) return;
  SubTile ta, tb;
  int ra, rb;
  uint32_t ha, hb;
  item(i, ra, ha);
  load_subtile(ta, kg, vg, ra, ha ? row_end : ra, lane);
  // issues the loads of item j into t (unconditional, so the compiler keeps them in flight
  // over the compute that follows); past the last item, or for an item no head needs,
  // every lane reads one row (512 B)
  auto next = [&](int j, SubTile& t, int& r, uint32_t& h, int rcur) {
    r = rcur;
    h = 0;
    if (j < nitems) item(j, r, h);
    load_subtile(t, kg, vg, r, h ? row_end : r, lane);
  };
  while (true) {
    next(i + WAVES, tb, rb, hb, ra);
    attn_subtile<G>(s, ta, ra, row_end, ha, qk, scale_log2, lane);
    if (i + WAVES >= nitems) break;
    next(i + 2 * WAVES, ta, ra, ha, rb);
    attn_subtile<G>(s, tb, rb, row_end, hb, qk, scale_log2, lane);
    if (i + 2 * WAVES >= nitems) break;
    i += 2 * WAVES;
  }
}

// Sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48): gfx950's
// row-swap moves (v_permlane16_swap: rows 0 <-> 1 and 2 <-> 3; v_permlane32_swap:
// halves) on the VALU, without the LDS crossbar.  Every lane gets the same sum.
__device__ __forceinline__ float sum_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float s16 = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);  // row pair sum
  const uint32_t w = __float_as_uint(s16);
  const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Combine the per-lane state of every wave of the workgroup through LDS and leave,
// for head h and dim d, the normalised output and the natural-log LSE.
// sm/sl: [waves][G]; sacc: [waves][G][128].
template <int G, int WAVES>
__device__ __forceinline__ void attn_publish_wave(const AttnState<G>& s, float* sm, float* sl,
                                                  float* sacc, int wave, int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lt = wave_sumf(s.l[h]);
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = sum_rows(s.acc[h][k]);
    if (lane < 16) {
#pragma unroll
      for (int k = 0; k < 8; ++k) sacc[(wave * G + h) * kHeadDim + lane * 8 + k] = a[k];
    }
    if (lane == 0) {
      sm[wave * G + h] = s.m[h];
      sl[wave * G + h] = lt;
    }
  }
}

// After a barrier: merged (o[d], lse) of head h from the WAVES published states.
template <int G, int WAVES>
__device__ __forceinline__ void attn_merge(const float* sm, const float* sl, const float* sacc,
                                           int h, int d, float& o, float& lse) {
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm[w * G + h]);
  if (M == -INFINITY) {
    o = 0.f;
    lse = -INFINITY;
    return;
  }
  float L = 0.f, A = 0.f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const float f = fast_exp2(sm[w * G + h] - M);
    L = fmaf(sl[w * G + h], f, L);
    A = fmaf(sacc[(w * G + h) * kHeadDim + d], f, A);
  }
  o = A / L;
  lse = (M + __log2f(L)) * kLn2f;
}

}  // namespace rtp
