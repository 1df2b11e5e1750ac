// Calibration probes, not part of the path.
// rtp_stream_read: a plain read-only stream over a device buffer, the ceiling the path's
// HBM-bound kernels are compared with on the same part.  Every lane issues 16-byte loads
// (non-temporal, as the path's K/V and index-key streams use, or ordinary cached loads)
// over a grid-stride range and folds them into one word per workgroup, so no load can be
// dropped.
// rtp_mfma_rate: back-to-back v_mfma_f32_32x32x16_bf16 (the prefill's score MFMA) on four
// independent accumulators in every wave, the ceiling the MFMA-bound prefill is compared
// with.

#include "rtp_common.hpp"

namespace rtp {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = NT ? ld16_nt(reinterpret_cast<const uint16_t*>(src + i + u * stride)) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = NT ? ld16_nt(reinterpret_cast<const uint16_t*>(src + i)) : src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup (the fold keeps every load live)
  __shared__ uint32_t s_acc[kProbeThreads / kWave];
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int w = 0; w < kProbeThreads / kWave; ++w) a ^= s_acc[w];
    sink[blockIdx.x] = a;
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kMfmaThreads = 256;

// Every wave multiplies the same operand pieces (lane l: its 8 bf16 of A, then of B, from
// `ops`) into four accumulators; each thread writes the sum of its 64 accumulator elements.
// The operands' values matter for the rate: under constant operands the part holds a
// higher clock than under the bit patterns of real data.
__global__ __launch_bounds__(kMfmaThreads) void mfma_rate_kernel(const uint16_t* __restrict__ ops,
                                                                  float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ld16(ops + 8 * lane));
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, ld16(ops + 8 * (64 + lane)));
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  out[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = r;
}

}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" rtp_status rtp_mfma_rate(const void* ops, float* out, int n_workgroups, int iters, void* stream) {
  if (!ops || !out || ((uintptr_t)ops & 15)) return RTP_EINVAL;
  if (n_workgroups <= 0 || n_workgroups > 65535 || iters <= 0 || iters > 16384) return RTP_EINVAL;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(n_workgroups), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(ops), out, iters);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" rtp_status rtp_stream_read(const void* src, size_t bytes, unsigned int* sink, int n_workgroups,
                                      int nontemporal, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15)) return RTP_EINVAL;
  if (n_workgroups <= 0 || n_workgroups > 65535) return RTP_EINVAL;
  const size_t n16 = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(n_workgroups), dim3(kProbeThreads), 0, s,
                       static_cast<const uint4*>(src), n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(n_workgroups), dim3(kProbeThreads), 0, s,
                       static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}
