// Prefill: causal attention over a whole prompt (Review, Adaptive sparse attention:
// local heads keep the sliding window + sink rule in prefill as in decode, retrieval
// heads run full dense attention and so fill the full KV cache; Review, Efficiency &
// ultra-long robustness: the prefill sparsity is fixed in advance), and the prompt's
// low-rank index keys bf16(W^K_h k^pre) for the decode-time retrieval (Review, Adaptive
// sparse attention equation, the key side of s_h(m, n)).
//
// Attention is a flash-style MFMA kernel for gfx950.  A 512-thread workgroup takes 256
// queries of one head (32 per wave) and walks 64-key tiles: all tiles up to the
// diagonal for a retrieval head, the sink tiles and the window's tiles for a local head
// (the tiles in between are never loaded).  Each tile is copied to LDS once for all
// eight waves (four copy K, four copy V); the next tile's loads are in flight over this
// tile's compute.  Per tile and wave:
//   S^T = K Q^T   16 v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, the wave's
//                 queries held in registers as the B operand), so each lane's
//                 accumulators belong to one query: the online softmax needs only the
//                 lane's own values and one exchange with lane ^ 32;
//   O^T += V^T P^T  16 v_mfma_f32_32x32x16_f16: P^T straight from the S^T accumulators
//                 (rounded to fp16: p in [0, 1], 11 significant bits), V^T from LDS,
//                 where the tile is stored transposed and converted to fp16 once; each
//                 V^T row's 4-key quads sit at XOR-swizzled slots, so that within 16
//                 lanes neither the transposing stores (rows 8 apart) nor the operand
//                 reads (consecutive rows) meet twice in a bank pair.  The LDS has 64
//                 banks and serves 32 lanes of a b64 access at a time, so both still
//                 pair up two-way; a layout free of that as well (quad slots
//                 q ^ (r >> 1) ^ (r >> 3), stores alternating row parity by lane) took
//                 the conflict counter to zero but cost more VALU than it saved.
// The MFMAs of each block are scheduled with their LDS operand reads kReadAhead reads
// ahead (sched_group_barrier), the two score accumulators alternating.
// Products of bf16 q and k are exact in the fp32 accumulators; V goes to fp16 exactly
// for |v| in [2^-14, 65504] (smaller values keep an absolute error below 2^-25; larger
// ones are out of range).  Rows past a prompt's end are never read (loads clamp to its
// last row) and never written.

#include "rtp_common.hpp"

namespace rtp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfM = 32 * kPfWaves;        // queries per workgroup
constexpr int kPfN = 64;                   // keys per tile
constexpr int kKStride = kHeadDim + 8;     // bf16 per K row in LDS (272 B: b128 reads spread over banks)
constexpr int kVStride = kPfN;             // fp16 per V^T row in LDS (128 B; banks spread by the quad swizzle)
constexpr int kReadAhead = 6;             // LDS operand reads in flight ahead of the MFMAs

struct PrefillArgs {
  const uint16_t* q;  // bf16 [B, Hq, T, 128]
  const uint16_t* k;  // bf16 [B, Hkv, T, 128]
  const uint16_t* v;  // bf16 [B, Hkv, T, 128]
  const int* seq_lens;
  const int* ret_heads;
  float* out;         // fp32 [B, Hq, T, 128]
  int Hq, Hkv, n_ret, T, window, sinks, n_mtiles;
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float max_pair(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float sum_pair(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Slot of key quad q (keys 4q .. 4q + 3 of the tile) in V^T row r (dim r): q XOR a
// function of r that differs between any 16 consecutive rows and between rows 8 apart.
__device__ __forceinline__ int vslot(int r, int q) { return (q ^ (r >> 3) ^ r) & 15; }

// two waves per SIMD: at most 256 VGPRs a wave
__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[kPfN * kKStride];
  __shared__ __attribute__((aligned(16))) _Float16 sv[kHeadDim * kVStride];
  // Workgroups go to the 8 XCDs round-robin by linear id (x + Hq y + ...), so a fixed
  // x -> head map would put a retrieval head's (heavier, causal) workgroups on the same
  // XCD in every row; rotating the map by the row spreads them over all XCDs.
  const int G = a.Hq / a.Hkv;
  const int h = ((int)blockIdx.x + (int)blockIdx.y) % a.Hq, g = h / G, b = blockIdx.z;
  const int mt = a.n_mtiles - 1 - (int)blockIdx.y;  // the late (heavy) query tiles first
  const int N = a.seq_lens[b];
  const int m0 = mt * kPfM;
  if (m0 >= N) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5;
  bool ret = false;  // is h a retrieval head
  for (int i0 = 0; i0 < a.n_ret; i0 += kWave) {
    const int i = i0 + lane;
    ret |= __ballot(i < a.n_ret && a.ret_heads[i] == h) != 0;
  }
  const int S = a.sinks, W = a.window;

  // key tiles: [r0b, r0e) then [r1b, r1e)
  const int qlast = min(m0 + kPfM, N) - 1;
  const int kt_end = qlast / kPfN + 1;
  int r0e = kt_end, r1b = 0, r1e = 0;
  if (!ret) {
    const int se = min(ceil_div(S, kPfN), kt_end);  // tiles holding sinks
    if (W == 0) {
      r0e = se;
    } else {
      const int ws = max(0, m0 + 1 - W) / kPfN;       // first tile of the earliest query's window
      if (ws > se) {
        r0e = se;
        r1b = ws;
        r1e = kt_end;
      }
    }
  }
  const int n0 = r0e, ntiles = r0e + (r1e - r1b);

  const size_t kvoff = ((size_t)b * a.Hkv + g) * (size_t)a.T * kHeadDim;
  const uint16_t* __restrict__ kbase = a.k + kvoff;
  const uint16_t* __restrict__ vbase = a.v + kvoff;

  // this wave's queries; lane holds query qw0 + (lane & 31) (row clamped for loading)
  const int qw0 = m0 + 32 * wave, qw1 = qw0 + 31;
  const int qi = qw0 + (lane & 31);
  uint4 qreg[8];
  {
    const uint16_t* qrow = a.q + (((size_t)b * a.Hq + h) * a.T + min(qi, N - 1)) * kHeadDim + 8 * hi;
#pragma unroll
    for (int c = 0; c < 8; ++c) qreg[c] = ld16(qrow + 16 * c);
    // the query rows are waited for here, once: otherwise the compiler's wait for them
    // inside the loop (vector loads retire in order) would also wait for the next tile's
    // loads issued just before each tile's MFMAs
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("" ::"v"(qreg[c].x), "v"(qreg[c].y), "v"(qreg[c].z), "v"(qreg[c].w));
  }

  // tile copies: waves 4-7 move K (1024 chunks of 16 B, 4 a thread); waves 0-3 move V,
  // thread (dim chunk dc = ct % 16, key quad kq = ct / 16) taking dims 8 dc .. 8 dc + 7 of
  // keys 4 kq .. 4 kq + 3 (16 lanes read one 256-byte row), stored transposed in fp16
  constexpr int kCopy = kPfThreads / 2;
  const bool do_k = tid >= kCopy, do_v = tid < kCopy;
  const int ct = tid & (kCopy - 1);
  const int dc = ct & 15, kq = ct >> 4;
  uint4 kreg[4], vreg[4];
  auto tile_of = [&](int t) { return t < n0 ? t : r1b + (t - n0); };
  auto gload = [&](int t) {
    const int key0 = tile_of(t) * kPfN;
    if (do_k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = ct + e * kCopy;  // row ch / 16, column ch % 16
        const int key = min(key0 + (ch >> 4), N - 1);
        kreg[e] = ld16(kbase + (size_t)key * kHeadDim + (ch & 15) * 8);
      }
    }
    if (do_v) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = min(key0 + 4 * kq + e, N - 1);
        vreg[e] = ld16(vbase + (size_t)key * kHeadDim + dc * 8);
      }
    }
  };
  auto lstore = [&]() {
    if (do_k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = ct + e * kCopy;
        *reinterpret_cast<uint4*>(&sk[(ch >> 4) * kKStride + (ch & 15) * 8]) = kreg[e];
      }
    }
    if (do_v) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        f16x4_t hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = word(vreg[e], d >> 1);
          hv[e] = (_Float16)((d & 1) ? bf_hi(w) : bf_lo(w));
        }
        const int r = dc * 8 + d;
        *reinterpret_cast<f16x4_t*>(&sv[r * kVStride + 4 * vslot(r, kq)]) = hv;
      }
    }
  };

  f32x16_t acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = (float)(kLog2e / 11.313708498984761);  // log2(e) / sqrt(128)

  if (ntiles > 0) gload(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // the previous tile's LDS reads are done
    lstore();
    __syncthreads();
    if (t + 1 < ntiles) gload(t + 1);  // in flight over this tile's compute

    const int key0 = tile_of(t) * kPfN, key1 = key0 + kPfN - 1;
    // wave-uniform: skip a tile no query of this wave attends to; mask only at edges
    const bool skip = qw0 >= N || key0 > qw1 || (!ret && key0 >= S && key1 <= qw0 - W);
    if (!skip) {
      const bool full = key1 <= qw0 && (ret || key1 < S || key0 > qw1 - W);
      const uint16_t* skb = sk;
      const _Float16* svb = sv;

      f32x16_t s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const uint16_t* krow = &skb[(32 * sb + (lane & 31)) * kKStride + 8 * hi];
          const uint4 kv = *reinterpret_cast<const uint4*>(krow + 16 * c);
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                           __builtin_bit_cast(bf16x8_t, qreg[c]), s[sb], 0, 0, 0);
        }
      }
      // schedule: the K operand reads run kReadAhead reads ahead of the MFMAs (masks:
      // 0x100 LDS reads, 0x008 MFMA), so an MFMA rarely waits on the LDS
      __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);
#pragma unroll
      for (int i = 0; i < 16 - kReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 0);
      // lane's scores: key key0 + 32 sb + 8 (r / 4) + 4 hi + r % 4, query qi (raw q.k)
      // masks as compares of the element's compile-time key offset c (key = kb + c) with
      // three per-lane bounds: key <= qi, key < S (sink), key > qi - W (window)
      float mt_ = -INFINITY;
      if (full) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt_ = fmaxf(mt_, s[sb][r]);
      } else {
        const int kb = key0 + 4 * hi;
        const int d_causal = qi - kb, d_win = qi - W - kb, d_sink = S - kb;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * sb + 8 * (r >> 2) + (r & 3);
            const bool ok = (c <= d_causal) & (ret | (c < d_sink) | (c > d_win));
            s[sb][r] = ok ? s[sb][r] : -INFINITY;
            mt_ = fmaxf(mt_, s[sb][r]);
          }
      }
      mt_ = max_pair(mt_);
      // rescale only when some query's maximum grew (wave-uniform branch); elsewhere the
      // factor would be exactly 1
      if (__ballot(mt_ > m_run) != 0) {
        const float m_new = fmaxf(m_run, mt_);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * scale);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
      }
      // p = 2^((s - m) scale); nothing attended yet (m = -inf): p = 0 for every key
      const float msc = m_run == -INFINITY ? 0.f : m_run * scale;
      float ls = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[sb][r], scale, -msc));
          s[sb][r] = p;
          ls += p;
        }
      l_run += ls;
      // P^T operand of chunk c: keys 16 c + 4 hi + 0..3 and 16 c + 8 + 4 hi + 0..3
      f16x8_t pb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < 8; ++u) pb[c][u] = (_Float16)s[c >> 1][8 * (c & 1) + u];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int r = 32 * d + (lane & 31);
          const _Float16* vrow = &svb[r * kVStride];
          const f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vrow + 4 * vslot(r, 4 * c + hi));
          const f16x4_t up = *reinterpret_cast<const f16x4_t*>(vrow + 4 * vslot(r, 4 * c + 2 + hi));
          const f16x8_t av = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[c], acc[d], 0, 0, 0);
        }
      }
      // the same for the V operand reads, two per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kReadAhead, 1);
#pragma unroll
      for (int i = 0; i < 16 - kReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 1);
    }
  }

  // lanes l and l ^ 32 hold the two halves of query qi's keys; both have m_run
  const float lt = sum_pair(l_run);
  if (qi >= N) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  float* orow = a.out + (((size_t)b * a.Hq + h) * a.T + qi) * kHeadDim;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 o = make_float4(acc[d][4 * q4] * inv, acc[d][4 * q4 + 1] * inv, acc[d][4 * q4 + 2] * inv,
                                   acc[d][4 * q4 + 3] * inv);
      *reinterpret_cast<float4*>(orow + 32 * d + 8 * q4 + 4 * hi) = o;
    }
}

// ---------------------------------------------------------------- prompt index keys
constexpr int kKeyThreads = 256;
constexpr int kKeyRows = 64;  // prompt rows per workgroup

struct KeyArgs {
  const uint16_t* k_pre;  // bf16 [B, Hkv, T, 128]
  const uint16_t* w_k;    // bf16 [n_ret, 16, 128]
  const int* seq_lens;
  const int* ret_heads;
  uint16_t* k_idx;        // bf16 [B, n_ret, T, 16]
  int Hq, Hkv, n_ret, T;
};

// Thread (i, part): output dim i = tid / 16 of every row, over dims 8 part .. 8 part + 7;
// its W^K_h slice stays in registers.  The exact sum of the 128 products is rounded once
// to bf16 (index_key_bf16), as the decode-side append does.
__global__ __launch_bounds__(kKeyThreads) void prompt_keys_kernel(KeyArgs a) {
  const int r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int N = a.seq_lens[b];
  const int row0 = blockIdx.x * kKeyRows;
  if (row0 >= N) return;
  const int i = tid >> 4, part = tid & 15;
  const int g = a.ret_heads[r] / (a.Hq / a.Hkv);
  const uint4 wv = ld16(a.w_k + ((size_t)r * kIndexDim + i) * kHeadDim + part * 8);
  const uint16_t* kp = a.k_pre + ((size_t)b * a.Hkv + g) * (size_t)a.T * kHeadDim + part * 8;
  uint16_t* ko = a.k_idx + ((size_t)b * a.n_ret + r) * (size_t)a.T * kIndexDim + i;
  const int row1 = min(row0 + kKeyRows, N);
  for (int row = row0; row < row1; ++row) {  // uniform trip count: the DPP sums see every lane
    const uint4 kv = ld16(kp + (size_t)row * kHeadDim);
    const uint32_t key = index_key_bf16(wv, kv);
    if (part == 0) ko[(size_t)row * kIndexDim] = (uint16_t)key;
  }
}

}  // namespace
}  // namespace rtp

using namespace rtp;

extern "C" rtp_status rtp_prefill_attn(const void* q, const void* k, const void* v, const int* seq_lens,
                                       const int* ret_heads, int B, int Hq, int Hkv, int n_ret, int max_ctx,
                                       int window, int sinks, float* out, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (n_ret < Hq && (window < 0 || sinks < 0 || window + sinks < 1)) return RTP_EINVAL;
  if (!q || !k || !v || !seq_lens || !out || (n_ret > 0 && !ret_heads)) return RTP_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return RTP_EINVAL;
  const int n_mtiles = ceil_div(max_ctx, kPfM);
  if (n_mtiles > 65535 || Hq > 65535 || B > 65535) return RTP_EUNSUPPORTED;
  const PrefillArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                      static_cast<const uint16_t*>(v), seq_lens, ret_heads, out, Hq, Hkv, n_ret, max_ctx,
                      n_ret < Hq ? window : 0, n_ret < Hq ? sinks : 0, n_mtiles};
  hipLaunchKernelGGL(prefill_kernel, dim3(Hq, n_mtiles, B), dim3(kPfThreads), 0, static_cast<hipStream_t>(stream),
                     a);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}

extern "C" rtp_status rtp_prefill_index_keys(const void* k_pre, const void* w_k, const int* seq_lens,
                                             const int* ret_heads, int B, int Hq, int Hkv, int n_ret, int max_ctx,
                                             void* k_idx, void* stream) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_ret < 0 || n_ret > Hq || max_ctx <= 0) return RTP_EINVAL;
  if (Hq % Hkv) return RTP_EINVAL;
  if (n_ret == 0) return RTP_OK;
  if (!k_pre || !w_k || !seq_lens || !ret_heads || !k_idx) return RTP_EINVAL;
  if ((((uintptr_t)k_pre | (uintptr_t)w_k) & 15) || ((uintptr_t)k_idx & 1)) return RTP_EINVAL;
  const int nx = ceil_div(max_ctx, kKeyRows);
  if (n_ret > 65535 || B > 65535) return RTP_EUNSUPPORTED;
  const KeyArgs a{static_cast<const uint16_t*>(k_pre), static_cast<const uint16_t*>(w_k), seq_lens, ret_heads,
                  static_cast<uint16_t*>(k_idx), Hq, Hkv, n_ret, max_ctx};
  hipLaunchKernelGGL(prompt_keys_kernel, dim3(nx, n_ret, B), dim3(kKeyThreads), 0, static_cast<hipStream_t>(stream),
                     a);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ELAUNCH;
}
