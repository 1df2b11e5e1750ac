// Calibration probe, not part of the decode path: a plain read-only stream over a device
// buffer, the ceiling the path's HBM-bound kernels are compared with on the same part.
// Every lane issues 16-byte loads (non-temporal, as the path's K/V and index-key streams
// use, or ordinary cached loads) over a grid-stride range and folds them into one word
// per workgroup, so no load can be dropped.

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

}  // namespace
}  // namespace rtp

using namespace rtp;

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
