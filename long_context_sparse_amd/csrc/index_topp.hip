// Kernel 1 of the decode path as its own launch: low-rank index scoring and exact
// block top-p (the device code and its description are in rtp_index.hpp).
//
// gfx950 launch: grid (chunk, retrieval head, sequence), 1024 threads = 16 wave64; the
// chunks are sized for about one workgroup per compute unit, so the scoring runs in a
// single wave of workgroups; a larger grid (many heads with long sequences) gets a build
// that fits two workgroups per unit.  The selecting workgroup of each head runs its passes over blocks
// on all 16 waves and its serial steps on one.  Each head's tag word lives in its workspace region and is advanced
// by the head's selecting workgroup at the end of every call.

#include "rtp_index.hpp"

namespace rtp {
namespace {

constexpr int kIdxThreads = 1024;

static_assert(kIdxMaxChunks % kIdxThreads == 0, "chunk words per thread");

struct K1Layout {
  IndexGeom g;
  size_t stride, total;
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

// The workspace: the header, then one region per head whose size depends only on the
// blocks per sequence (room for the most chunks a head can have), so neither the size
// of a region nor where it starts depends on the device; `target` (workgroups wanted)
// sets one launch's chunking.
K1Layout k1_layout(int B, int n_ret, int max_ctx, int block, int target) {
  K1Layout L{};
  L.g = index_geom(B, n_ret, max_ctx, block, kIdxThreads, target);
  L.stride = index_head_stride(L.g.nblk_max);
  L.total = kIdxWsHeaderBytes + (size_t)B * n_ret * L.stride;
  return L;
}

// One index workgroup: chunk c of head (b, r); the last of the head to finish selects.
template <int BK, int WPS>
__device__ __forceinline__ void index_role(const IndexArgs& a, int c, int r, int b, unsigned char* smem) {
  auto* S = reinterpret_cast<IndexSmem<kIdxThreads>*>(smem);
  const size_t head = (size_t)b * a.n_ret + r;
  if (!index_chunk<BK, kIdxThreads>(a, c, r, b, S)) return;
  index_select<kIdxThreads, WPS>(a, BK, b, head, S);
  index_advance_tag<kIdxThreads>(a, head, S->tag);
}

// Grid z is a rank, not a sequence: the workgroups of rank z serve the sequence with the
// z-th most tokens (ties by index), so a ragged batch's longest sequences, whose chunks and
// selections take longest, are dispatched first and the grid ends on the short ones.
// Every workgroup ranks the lengths itself (one round of loads; batches over
// kIdxOrderMax keep the index order).
constexpr int kIdxOrderMax = 256;

__device__ __forceinline__ int index_seq_of_rank(const int* __restrict__ seq_lens, int rank) {
  const int B = gridDim.z;
  if (B == 1 || B > kIdxOrderMax) return rank;
  __shared__ int s_len[kIdxOrderMax];
  __shared__ int s_seq;
  const int t = threadIdx.x;
  if (t < B) s_len[t] = seq_lens[t];
  __syncthreads();
  if (t < B) {
    const int lt = s_len[t];
    int rk = 0;
    for (int j = 0; j < B; ++j) {
      const int lj = s_len[j];
      rk += (lj > lt) | ((lj == lt) & (j < t));
    }
    if (rk == rank) s_seq = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_seq);
}

// WPS = waves a SIMD must hold: 4 (one workgroup per compute unit, the registers the
// code wants) for grids of at most one workgroup per unit, 8 (two workgroups per unit,
// at most 64 VGPRs with a few spilled) for larger grids, whose later workgroups then
// start while a unit's first one is still scoring or selecting.
template <int BK, int WPS>
__global__ __launch_bounds__(kIdxThreads, WPS) void index_topp_kernel(IndexArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // Workgroups go to the XCDs round-robin by linear id, so with chunk = x a chunk index
  // would land on the same XCD for every head, and a ragged batch (whose short sequences
  // have only their first chunks) would load the XCDs of the low chunk indices most; the
  // chunk index is rotated by the head and sequence instead.
  const int c = (int)((blockIdx.x + blockIdx.y + (size_t)blockIdx.z * gridDim.y) % gridDim.x);
  index_role<BK, WPS>(a, c, blockIdx.y, index_seq_of_rank(a.seq_lens, blockIdx.z), smem_raw);
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

// Checks kernel 1's arguments (n_ret > 0) and fills its arguments, grid and LDS size, with
// either selection rule: top_p per head (topk_blocks == 0) or a fixed number of blocks per
// head (topk_blocks > 0).
rtp_status index_prepare(const void* q_pre, const void* w_q, const void* k_idx, const int* seq_lens,
                         const int* ret_heads, const float* top_p, int topk_blocks, int B, int Hq, int n_ret,
                         int max_ctx, int block, int* sel_idx, int* sel_cnt, unsigned char* sel_mask,
                         void* workspace, size_t ws_bytes, IndexArgs& args, dim3& grid, size_t& dyn) {
  if (!q_pre || !w_q || !k_idx || !seq_lens || !ret_heads || (topk_blocks == 0 && !top_p) || !sel_idx ||
      !sel_cnt || !workspace)
    return RTP_EINVAL;
  if (((uintptr_t)q_pre | (uintptr_t)w_q | (uintptr_t)k_idx) & 15) return RTP_EINVAL;
  if ((uintptr_t)workspace & 255) return RTP_EINVAL;
  if (ws_bytes < k1_layout(B, n_ret, max_ctx, block, 1).total) return RTP_EINVAL;
  const K1Layout L = k1_layout(B, n_ret, max_ctx, block, compute_units());
  char* ws = static_cast<char*>(workspace);
  args = IndexArgs{static_cast<const uint16_t*>(q_pre), static_cast<const uint16_t*>(w_q),
                   static_cast<const uint16_t*>(k_idx), seq_lens, ret_heads, topk_blocks ? nullptr : top_p,
                   topk_blocks, Hq, n_ret, max_ctx, L.g.nblk_max, L.g.chunk_blocks, index_chunk_cap(L.g.nblk_max),
                   sel_idx, sel_cnt, sel_mask, reinterpret_cast<IndexWsHeader*>(ws), ws + kIdxWsHeaderBytes,
                   L.stride};
  grid = dim3(L.g.n_chunk, n_ret, B);
  dyn = index_smem_bytes<kIdxThreads>(L.g.rows);
  return RTP_OK;
}

rtp_status index_scalar_check(int B, int Hq, int n_ret, int max_ctx, int block) {
  if (B <= 0 || Hq <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (block != 64 && block != 128) return RTP_EUNSUPPORTED;
  if (ceil_div(max_ctx, block) > kIdxMaxBlocks) return RTP_EUNSUPPORTED;
  if (B > 65535 || n_ret > 65535) return RTP_EUNSUPPORTED;
  return RTP_OK;
}

// Checks the arguments and enqueues kernel 1 alone.
rtp_status index_launch(const void* q_pre, const void* w_q, const void* k_idx, const int* seq_lens,
                        const int* ret_heads, const float* top_p, int topk_blocks, int B, int Hq, int n_ret,
                        int max_ctx, int block, int* sel_idx, int* sel_cnt, unsigned char* sel_mask,
                        void* workspace, size_t ws_bytes, void* stream) {
  const rtp_status sc = index_scalar_check(B, Hq, n_ret, max_ctx, block);
  if (sc != RTP_OK) return sc;
  if (n_ret == 0) return RTP_OK;
  IndexArgs args{};
  dim3 grid;
  size_t dyn = 0;
  const rtp_status st = index_prepare(q_pre, w_q, k_idx, seq_lens, ret_heads, top_p, topk_blocks, B, Hq, n_ret,
                                      max_ctx, block, sel_idx, sel_cnt, sel_mask, workspace, ws_bytes, args, grid,
                                      dyn);
  if (st != RTP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool one_wave = (long long)grid.x * grid.y * grid.z <= compute_units();
  if (block == 64) {
    if (one_wave)
      hipLaunchKernelGGL((index_topp_kernel<64, 4>), grid, dim3(kIdxThreads), dyn, s, args);
    else
      hipLaunchKernelGGL((index_topp_kernel<64, 8>), grid, dim3(kIdxThreads), dyn, s, args);
  } else {
    if (one_wave)
      hipLaunchKernelGGL((index_topp_kernel<128, 4>), grid, dim3(kIdxThreads), dyn, s, args);
    else
      hipLaunchKernelGGL((index_topp_kernel<128, 8>), grid, dim3(kIdxThreads), dyn, s, args);
  }
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
