// Kernel 1 of the decode path as its own launch: low-rank index scoring and exact
// block top-p (the device code and its description are in rtp_index.hpp).
//
// gfx950 launch: grid (chunk, retrieval head, sequence), 1024 threads = 16 wave64, one
// workgroup per compute unit at a time (its registers and LDS allow one), so the chunks
// are sized for about one workgroup per compute unit and the scoring runs in a single
// wave of workgroups; the selecting workgroup of each head then has 16 waves for the
// threshold search.  Each head's tag word lives in the workspace and is advanced by the
// head's selecting workgroup at the end of every call.

#include "rtp_index.hpp"

namespace rtp {
namespace {

constexpr int kIdxThreads = 1024;

constexpr int kIdxMaxChunks = 2 * kIdxThreads;  // chunks per head the selection combines

struct K1Layout {
  IndexGeom g;
  size_t off_counters, off_tag, off_cmax, off_e, total;
};

// Compute units of the current device (cached per device; 256, MI355X's count, if it
// cannot be queried).
int compute_units() {
  static thread_local int cached_dev = -1, cached_n = 256;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    cached_n = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    cached_dev = dev;
  }
  return cached_n;
}

// The workspace has room for the most chunks a head can have, so its size does not
// depend on the device; `target` (workgroups wanted) sets one launch's chunking.
K1Layout k1_layout(int B, int n_ret, int max_ctx, int block, int target) {
  K1Layout L{};
  L.g = index_geom(B, n_ret, max_ctx, block, kIdxThreads, target);
  const size_t heads = (size_t)B * n_ret;
  L.off_counters = 0;
  L.off_tag = align_up(heads * sizeof(int), 256);
  L.off_cmax = L.off_tag + align_up(heads * sizeof(uint32_t), 256);
  L.off_e = L.off_cmax + align_up(heads * kIdxMaxChunks * 2 * sizeof(uint64_t), 256);
  L.total = L.off_e + align_up(heads * (size_t)L.g.nblk_max * sizeof(uint64_t), 256);
  return L;
}

template <int BK>
__global__ __launch_bounds__(kIdxThreads) void index_topp_kernel(IndexArgs a, uint32_t* __restrict__ tags) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  auto* S = reinterpret_cast<IndexSmem<kIdxThreads>*>(smem_raw);
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const size_t head = (size_t)b * a.n_ret + r;
  if (!index_chunk<BK, kIdxThreads>(a, c, r, b, tags + head, S)) return;
  index_select<kIdxThreads>(a, BK, r, b, S);
  if (threadIdx.x == 0)
    __hip_atomic_store(&tags[head], next_tag(S->tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" size_t rtp_index_topp_workspace_size(int B, int n_ret, int max_ctx, int block) {
  if (B <= 0 || n_ret <= 0 || max_ctx <= 0 || (block != 64 && block != 128)) return 0;
  if (ceil_div(max_ctx, block) > kIdxMaxBlocks) return 0;
  return k1_layout(B, n_ret, max_ctx, block, 1).total;
}

namespace {

// Checks the arguments and enqueues kernel 1 with either selection rule: top_p per head
// (topk_blocks == 0) or a fixed number of blocks per head (topk_blocks > 0).
rtp_status index_launch(const void* q_pre, const void* w_q, const void* k_idx, const int* seq_lens,
                        const int* ret_heads, const float* top_p, int topk_blocks, int B, int Hq, int n_ret,
                        int max_ctx, int block, int* sel_idx, int* sel_cnt, unsigned char* sel_mask,
                        void* workspace, size_t ws_bytes, void* stream) {
  if (B <= 0 || Hq <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
  if (ceil_div(max_ctx, block) > kIdxMaxBlocks) return RTP_EUNSUPPORTED;
  if (B > 65535 || n_ret > 65535) return RTP_EUNSUPPORTED;
  if (n_ret == 0) return RTP_OK;
  if (!q_pre || !w_q || !k_idx || !seq_lens || !ret_heads || (topk_blocks == 0 && !top_p) || !sel_idx ||
      !sel_cnt || !workspace)
    return RTP_EINVAL;
  if (((uintptr_t)q_pre | (uintptr_t)w_q | (uintptr_t)k_idx) & 15) return RTP_EINVAL;
  if ((uintptr_t)workspace & 255) return RTP_EINVAL;
  if (ws_bytes < k1_layout(B, n_ret, max_ctx, block, 1).total) return RTP_EINVAL;
  const K1Layout L = k1_layout(B, n_ret, max_ctx, block, compute_units());
  char* ws = static_cast<char*>(workspace);
  IndexArgs args{static_cast<const uint16_t*>(q_pre), static_cast<const uint16_t*>(w_q),
                 static_cast<const uint16_t*>(k_idx), seq_lens, ret_heads, topk_blocks ? nullptr : top_p,
                 topk_blocks, Hq, n_ret, max_ctx, L.g.nblk_max, L.g.chunk_blocks, kIdxMaxChunks, sel_idx, sel_cnt,
                 sel_mask, reinterpret_cast<int*>(ws + L.off_counters), reinterpret_cast<uint64_t*>(ws + L.off_cmax),
                 reinterpret_cast<uint64_t*>(ws + L.off_e)};
  uint32_t* tags = reinterpret_cast<uint32_t*>(ws + L.off_tag);
  dim3 grid(L.g.n_chunk, n_ret, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t dyn = index_smem_bytes<kIdxThreads>(L.g.rows);
  if (block == 64)
    hipLaunchKernelGGL(index_topp_kernel<64>, grid, dim3(kIdxThreads), dyn, s, args, tags);
  else
    hipLaunchKernelGGL(index_topp_kernel<128>, grid, dim3(kIdxThreads), dyn, s, args, tags);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

}  // namespace

extern "C" rtp_status rtp_index_topp(const void* q_pre, const void* w_q, const void* k_idx,
                                     const int* seq_lens, const int* ret_heads, const float* top_p,
                                     int B, int Hq, int n_ret, int max_ctx, int block, int* sel_idx,
                                     int* sel_cnt, unsigned char* sel_mask, void* workspace, size_t ws_bytes,
                                     void* stream) {
  return index_launch(q_pre, w_q, k_idx, seq_lens, ret_heads, top_p, 0, B, Hq, n_ret, max_ctx, block, sel_idx,
                      sel_cnt, sel_mask, workspace, ws_bytes, stream);
}

extern "C" rtp_status rtp_index_topk(const void* q_pre, const void* w_q, const void* k_idx,
                                     const int* seq_lens, const int* ret_heads, int k_tokens,
                                     int B, int Hq, int n_ret, int max_ctx, int block, int* sel_idx,
                                     int* sel_cnt, unsigned char* sel_mask, void* workspace, size_t ws_bytes,
                                     void* stream) {
  if (k_tokens <= 0) return RTP_EINVAL;
  if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
  const int kb = (int)(((long long)k_tokens + block - 1) / block);
  return index_launch(q_pre, w_q, k_idx, seq_lens, ret_heads, nullptr, kb, B, Hq, n_ret, max_ctx, block, sel_idx,
                      sel_cnt, sel_mask, workspace, ws_bytes, stream);
}
