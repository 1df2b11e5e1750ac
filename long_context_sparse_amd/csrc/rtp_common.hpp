// Device helpers shared by the gfx950 kernels of librtp.so (wave64 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtp.h"

namespace rtp {

constexpr int kHeadDim = RTP_HEAD_DIM;
constexpr int kIndexDim = RTP_INDEX_DIM;
constexpr int kWave = 64;

constexpr double kLog2e = 1.4426950408889634073599246810019;
constexpr float kLn2f = 0.69314718055994530941723212145818f;

// bf16 pair packed in one dword -> the two fp32 values (exact).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Cross-lane moves on the VALU (DPP, gfx9 controls), no LDS traffic.  Every lane's
// source is inside its row, so no lane reads out of range.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16 lanes
constexpr int kDppRowBcast0 = 0x150;  // + n: every lane <- lane n of its 16-lane row

// (every lane is written, so the destination's old value is never needed)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Wave-wide reductions: a butterfly within each row of 16 lanes (after it every lane of
// a row holds the same row result), then the four rows combined in a fixed order, so
// the result is identical in every lane and independent of the lane order.
template <class T, class Op>
__device__ __forceinline__ T wave_reduce_dpp(T v, Op op) {
  if constexpr (sizeof(T) == 8) {
    v = op(v, dpp_f64<kDppXor1>(v));
    v = op(v, dpp_f64<kDppXor2>(v));
    v = op(v, dpp_f64<kDppHalfMirror>(v));
    v = op(v, dpp_f64<kDppMirror>(v));
    return op(op(readlane_f64(v, 0), readlane_f64(v, 16)), op(readlane_f64(v, 32), readlane_f64(v, 48)));
  } else {
    v = op(v, dpp_f32<kDppXor1>(v));
    v = op(v, dpp_f32<kDppXor2>(v));
    v = op(v, dpp_f32<kDppHalfMirror>(v));
    v = op(v, dpp_f32<kDppMirror>(v));
    return op(op(readlane_f32(v, 0), readlane_f32(v, 16)), op(readlane_f32(v, 32), readlane_f32(v, 48)));
  }
}

// Inclusive prefix sums over the 64 lanes of a wave: a Hillis-Steele scan inside each
// 16-lane row on DPP row shifts (a lane whose source lies before its row's start adds
// 0), then each row adds the totals of the rows below it, read from lanes 15, 31, 47.
constexpr int kDppRowShr = 0x110;  // + n: lane i <- lane i - n of its row (n = 1..15)

template <int N>
__device__ __forceinline__ uint32_t dpp_shr_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr + N, 0xF, 0xF, false);
}
template <int N>
__device__ __forceinline__ uint64_t dpp_shr_u64(uint64_t v) {
  const uint32_t lo = dpp_shr_u32<N>((uint32_t)v), hi = dpp_shr_u32<N>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp_shr_u32<1>(x);
  x += dpp_shr_u32<2>(x);
  x += dpp_shr_u32<4>(x);
  x += dpp_shr_u32<8>(x);
  const uint32_t t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
                 t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

__device__ __forceinline__ double wave_max(double v) {
  return wave_reduce_dpp(v, [](double a, double b) { return fmax(a, b); });
}
__device__ __forceinline__ double wave_sum(double v) {
  return wave_reduce_dpp(v, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ float wave_maxf(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sumf(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return a + b; });
}

// 2^x on the hardware transcendental unit (no range reduction needed for decode logits).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// 16-byte global load of 8 bf16 values.
__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
// The same as a non-temporal (streaming) load, for data read once: it does not displace
// reusable lines from the caches, and streams read this way sustain a higher share of
// HBM bandwidth on gfx950 than cached loads.
__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// bf16 bit pattern of a double rounded once to nearest, ties to even: 8 significant
// bits, float32's exponent range, subnormals (quantum 2^-133) below 2^-126, infinity
// on overflow.
__device__ __forceinline__ uint32_t bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const int e = (int)((u >> 52) & 0x7FF);
  const uint64_t mant = u & ((1ull << 52) - 1ull);
  if (e == 0x7FF) return sign | 0x7F80u | (mant ? 0x40u : 0u);
  if (e == 0) return sign;                 // float64 subnormals: far below bf16's range
  const int eb = e - 1023 + 127;           // bf16 biased exponent of 1.m x 2^(e - 1023)
  const int s = eb > 0 ? 45 : 46 - eb;     // significant bits dropped (more when subnormal)
  if (s > 63) return sign;
  const uint64_t sig = (1ull << 52) | mant;
  uint32_t q = (uint32_t)(sig >> s);
  const uint64_t rem = sig & ((1ull << s) - 1ull), half = 1ull << (s - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  if (eb <= 0) return sign | q;            // q == 128 is the smallest normal's pattern
  int ebb = eb;
  if (q == 256u) {
    q = 128u;
    ++ebb;
  }
  if (ebb >= 255) return sign | 0x7F80u;
  return sign | ((uint32_t)ebb << 7) | (q - 128u);
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A wave-uniform 64-bit value moved to scalar registers; a 64-bit value of one lane.
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t b = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)b << 32) | a;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t a = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t b = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)b << 32) | a;
}
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
  x += dpp_shr_u64<1>(x);
  x += dpp_shr_u64<2>(x);
  x += dpp_shr_u64<4>(x);
  x += dpp_shr_u64<8>(x);
  const uint64_t t0 = readlane_u64(x, 15), t1 = readlane_u64(x, 31), t2 = readlane_u64(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0ull) + (row >= 2 ? t1 : 0ull) + (row >= 3 ? t2 : 0ull);
}

// ------------------------------------------------------------------ published words
// Values passed between workgroups of one launch without fences: every published
// 64-bit word carries the call's tag (1..4095, advanced by every call) in its low 12
// bits, words are written and read with relaxed device-scope atomics, and a reader
// re-reads a word until it carries the current tag.  An fp64 keeps its top 52 bits
// (relative precision 2^-40); an fp32 or an int sits in the high half.
constexpr uint64_t kTagBits = 0xFFFull;
constexpr int kSpinBudget = 1 << 12;  // re-reads a thread may spend waiting for one tag

__device__ __forceinline__ uint64_t tagged(double x, uint32_t tag) {
  return ((uint64_t)__double_as_longlong(x) & ~kTagBits) | tag;
}
__device__ __forceinline__ double untag(uint64_t w) { return __longlong_as_double((long long)(w & ~kTagBits)); }
__device__ __forceinline__ uint64_t tagged_f32(float x, uint32_t tag) {
  return ((uint64_t)__float_as_uint(x) << 32) | tag;
}
__device__ __forceinline__ float untag_f32(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool has_tag(uint64_t w, uint32_t tag) { return (uint32_t)(w & kTagBits) == tag; }
// Re-read a published word until it carries `tag` (bounded by the thread's budget).
__device__ __forceinline__ uint64_t settle(const uint64_t* p, uint64_t w, uint32_t tag, int& budget) {
  while (!has_tag(w, tag) && budget > 0) {
    --budget;
    __builtin_amdgcn_s_sleep(1);
    w = ld_dev(p);
  }
  return w;
}
// The tag a call uses, from the word that holds it (0 in a fresh workspace reads as 1),
// and the tag of the next call.
__device__ __forceinline__ uint32_t load_tag(const uint32_t* p) {
  const uint32_t t = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return t == 0 ? 1u : t;
}
__device__ __forceinline__ uint32_t next_tag(uint32_t t) { return t % 4095u + 1u; }

}  // namespace rtp
