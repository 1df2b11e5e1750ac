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

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// 2^x on the hardware transcendental unit (no range reduction needed for decode logits).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// 16-byte global load of 8 bf16 values.
__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace rtp
