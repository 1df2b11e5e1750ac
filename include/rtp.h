/*
 * rtp.h - C ABI of the MI355X (gfx950) decode-time sparse attention library
 * (librtp.so): RTPurbo's retrieval-head indexer with exact block top-p (or a static
 * top-k budget), block-sparse split attention with a cross-split log-sum-exp reduce,
 * and the local heads' sliding-window + sink attention; around that decode step, the
 * cache maintenance it needs (appending the decode token, sink + window rings for KV
 * groups without retrieval heads) and the prefill of a prompt (causal attention with
 * the same head split, the prompt's index keys, the rings' first fill).
 *
 * Sources (page title, section):
 *   Review        - the Korean paper review of RTPurbo (dongryeollee1.github.io),
 *                   "Method": "Adaptive sparse attention" (index score equation
 *                   s_h(m,n) = (W^Q_h q^pre)^T (W^K_h k^pre), S_h(m) = Top-P(s_h, p);
 *                   window + sink for local heads) and "Hardware-aware top-p decoding
 *                   kernel" (block-wise top-p, 256-bin histogram, last CTA finds the
 *                   threshold and writes the block mask, score and select fused).
 *   Strikes-Back  - "Full Attention Strikes Back: Transferring Full Attention into
 *                   Sparse within Hundred Training Steps" (aitrends.kr): method item 2
 *                   (O_h(m), a softmax of q.k/sqrt(d_h) over S_h(m)) and the
 *                   architecture paragraph (Kernel 1 at D16: per-block scoring and
 *                   histogram threshold; Kernel 2 at D128: block-sparse attention and a
 *                   cross-split reduce; atomic counters).
 *
 * Conventions shared by every call:
 *   - Fixed sizes: head_dim 128 (RTP_HEAD_DIM), index dim 16 (RTP_INDEX_DIM),
 *     KV block 64 or 128 tokens, query heads per KV head (Hq / Hkv) in {1, 2, 4, 8}.
 *   - Every tensor argument is a DEVICE pointer owned by the caller, contiguous,
 *     row-major, with the layout given at each argument.  bf16 tensors are passed as
 *     const void* (raw bf16 bits).  The library allocates nothing and keeps no global
 *     mutable state (except rtp_decode_step_noalloc's fixed device scratch and its per-
 *     device bookkeeping); it is reentrant for disjoint workspaces.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Each call
 *     checks its scalar arguments on the host (no device access, no synchronization),
 *     then enqueues its kernels on `stream` and returns.  Buffers must stay alive until
 *     the stream has passed the call.
 *   - Device-resident values (seq_lens, head lists, top_p) are preconditions and are
 *     not checked: 1 <= seq_lens[b] <= max_ctx, head ids in [0, Hq) and ascending, the
 *     retrieval and local lists disjoint, 0 < top_p.  Violations are undefined
 *     behaviour (a device fault surfaces at the caller's next synchronization).
 *   - Workspaces must be zero-filled once before their first use; the kernels return
 *     every counter in them to zero, so a workspace can be reused by later calls on
 *     the same stream (for the index workspace, see its header below).  Calls that
 *     share a workspace must not overlap.
 *   - Return codes: RTP_OK; RTP_EINVAL for a null pointer, a non-positive size, an
 *     inconsistent shape or a workspace that is too small; RTP_EUNSUPPORTED for a block
 *     size or head grouping outside the fixed set; RTP_ELAUNCH when HIP reports a
 *     launch error; RTP_ESCRATCH when rtp_decode_step_noalloc's sizes need more than its
 *     fixed scratch.  On any error nothing is enqueued, except for RTP_ELAUNCH.
 *   - n_ret == 0 (resp. n_loc == 0, n_heads == 0) is a no-op returning RTP_OK.
 */
#ifndef RTP_H_
#define RTP_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RTP_HEAD_DIM 128
#define RTP_INDEX_DIM 16

typedef enum {
  RTP_OK = 0,
  RTP_EINVAL = 1,
  RTP_EUNSUPPORTED = 2,
  RTP_ELAUNCH = 3,
  RTP_ESCRATCH = 4
} rtp_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* rtp_status_string(int status);

/* Library version string, e.g. "rtp 1.0 gfx950". */
const char* rtp_version(void);

/* Bytes of workspace rtp_index_topp needs for these sizes (0 if a size is invalid). */
size_t rtp_index_topp_workspace_size(int B, int n_ret, int max_ctx, int block);

/*
 * The index workspace (rtp_index_topp, rtp_index_topk) starts with this header; the
 * per-(sequence, retrieval head) state follows it, one region per head whose size
 * depends only on ceil(max_ctx / block).  So a workspace sized for the largest batch
 * serves every later call with fewer sequences or retrieval heads and the same number of
 * blocks per sequence.  The first call after the zero-fill stores that number in
 * `layout`; a later call with another number touches none of the state, selects every
 * block of every head (a superset of the top-p or top-k set) and sets
 * RTP_INDEX_LAYOUT_MISMATCH; such a call needs a freshly zero-filled workspace.
 *
 * The selecting workgroup of each head waits for the words the other workgroups of the
 * launch published (no fences; each word carries a 32-bit call tag), within a bounded
 * number of re-reads.  If a word is still stale when that bound runs out, the head's
 * selection falls back to every block and RTP_INDEX_WAIT_EXPIRED is set.  `status` is
 * sticky (the library never clears it) and `fallbacks` counts the heads that fell back;
 * the caller reads them from device memory when it wants to check (the library never
 * synchronizes), and may clear them between calls.  `inject` must stay 0: bit 0 makes
 * every bounded wait give up at once, for tests of the fallback.
 * A head's tag advances with every call; after 2^32 - 1 calls it restarts at 1, and
 * the head's words are cleared first, so a word written under an old tag is never taken
 * as current.
 */
#define RTP_INDEX_WAIT_EXPIRED 1u
#define RTP_INDEX_LAYOUT_MISMATCH 2u
typedef struct {
  unsigned int layout;    /* ceil(max_ctx / block) of the calls served; 0 in a fresh workspace */
  unsigned int status;    /* RTP_INDEX_* bits, sticky */
  unsigned int fallbacks; /* heads whose selection fell back to every block */
  unsigned int inject;    /* 0; bit 0: every bounded wait gives up (tests of the fallback) */
} rtp_index_ws_header;

/*
 * Kernel 1: low-rank index scoring + exact block top-p selection
 * (Review, Adaptive sparse attention equation and Hardware-aware top-p decoding
 * kernel; Strikes-Back architecture paragraph, Kernel 1 at D16).
 *
 * For each sequence b and retrieval head r (query head hq = ret_heads[r]):
 *   q_idx   = W^Q_r q_pre[b, hq]                          (fp64 on the device)
 *   s_n     = q_idx . k_idx[b, r, n]        for n < N = seq_lens[b]
 *   m_j     = sum_{n in block j} softmax_n(s)             (block j = tokens [j*block, (j+1)*block) ∩ [0, N))
 *   S       = the shortest prefix of the blocks ordered by m_j descending (ties by
 *             ascending j) whose cumulative mass reaches top_p[b, r]; every block
 *             when top_p >= 1 or no prefix reaches it.
 * The threshold is found exactly by a mass-weighted radix select over 256-bin LDS
 * histograms run by the last workgroup of each (b, r) to finish scoring (found with
 * an atomic counter), so scoring and selection are one launch.  Block masses carry
 * a relative error below 1e-6 against exact arithmetic.
 *
 *   q_pre     bf16 [B, Hq, 128]        pre-RoPE queries (rows ret_heads[] are read)
 *   w_q       bf16 [n_ret, 16, 128]    W^Q of each retrieval head
 *   k_idx     bf16 [B, n_ret, max_ctx, 16]  index keys W^K_r k_pre (rows >= N never read)
 *   seq_lens  int32 [B]                 N_b, 1 <= N_b <= max_ctx
 *   ret_heads int32 [n_ret]             query-head id of each retrieval head, ascending
 *   top_p     fp32 [B, n_ret]           0 < p; p >= 1 selects every block
 *   sel_idx   out int32 [B, n_ret, ceil(max_ctx / block)]  selected block ids,
 *             ascending, in the first sel_cnt[b, r] entries (the rest untouched)
 *   sel_cnt   out int32 [B, n_ret]      number of selected blocks (>= 1)
 *   sel_mask  optional out uint8 [B, n_ret, ceil(max_ctx / block)]: the same set as a block
 *             mask (Review, Hardware-aware top-p decoding kernel: the last workgroup writes
 *             the block mask), 1 = selected, 0 = not, for blocks < ceil(N_b / block) (the
 *             rest untouched); NULL to skip it
 *   workspace device scratch of >= rtp_index_topp_workspace_size(B, n_ret, max_ctx, block)
 *             bytes, zero-filled before first use, 256-byte aligned; it begins with an
 *             rtp_index_ws_header (above)
 */
rtp_status rtp_index_topp(const void* q_pre, const void* w_q, const void* k_idx,
                          const int* seq_lens, const int* ret_heads, const float* top_p,
                          int B, int Hq, int n_ret, int max_ctx, int block,
                          int* sel_idx, int* sel_cnt, unsigned char* sel_mask,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * Kernel 1 with the static top-k rule instead of top-p (Review, Experiments: the
 * fixed-budget variant with k = 4096 built to isolate the dynamic budget; Insight item 3
 * counts the budget in tokens): the same scores and block masses, and
 *   S = the ceil(k_tokens / block) blocks of largest m_j (ties by ascending j); every
 *       block when there are no more than that.
 * The same exact radix select finds the set, every block weighing 1.
 *
 *   k_tokens  budget in tokens, >= 1 (RTP_EINVAL otherwise)
 *   every other argument as in rtp_index_topp (same workspace)
 */
rtp_status rtp_index_topk(const void* q_pre, const void* w_q, const void* k_idx,
                          const int* seq_lens, const int* ret_heads, int k_tokens,
                          int B, int Hq, int n_ret, int max_ctx, int block,
                          int* sel_idx, int* sel_cnt, unsigned char* sel_mask,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * KV placement (Review, Method overview: only the retrieval heads need the full KV cache;
 * the other heads safely drop remote tokens).  With kv_slot (int32 [Hkv], device) the
 * KV groups live in two places:
 *   kv_slot[g] = s >= 0   full caches k_cache, v_cache  bf16 [B, n_full, max_ctx, 128],
 *                         group index s, position p at row p;
 *   kv_slot[g] = -1 - s   sink + window rings k_ring, v_ring  bf16 [B, n_ring, sinks + window,
 *                         128], group index s: position p < sinks at row p, a later position at
 *                         row sinks + (p - sinks) mod window (the last `window` positions are
 *                         kept; with window 0 nothing past the sinks).
 * The rings suit KV groups whose query heads are all local: their attention reads
 * exactly the sinks and the window.  n_full + n_ring <= Hkv (else RTP_EINVAL).  Slots
 * must be distinct and in range (device values, not checked).  kv_slot NULL: every group
 * is in the full caches at its own index.
 */

/*
 * Kernel 2: block-sparse exact attention over the selected blocks, split along the
 * context (Strikes-Back method item 2, O_h(m) with the value vector; architecture
 * paragraph, Kernel 2 at D128).
 *
 * For each sequence b, retrieval head r (query head hq, KV head g = hq / (Hq/Hkv))
 * and context split c (blocks [c*split_tokens/block, (c+1)*split_tokens/block)):
 *   T_c = tokens n < N of the blocks in sel_idx[b, r, :sel_cnt[b, r]] that fall in c
 *   o_part[b, r, c]   = sum_{n in T_c} softmax_n(q[b,hq] . K[b,g,n] / sqrt(128)) V[b,g,n]
 *   lse_part[b, r, c] = log sum_{n in T_c} exp(q[b,hq] . K[b,g,n] / sqrt(128))
 * with o = 0 and lse = -inf for an empty T_c.  One workgroup serves every retrieval
 * head of a KV group, so a block selected by several heads of the group is read once.
 *
 *   q          bf16 [B, Hq, 128]        queries (post-RoPE)
 *   k_cache    bf16 [B, Hkv, max_ctx, 128]
 *   v_cache    bf16 [B, Hkv, max_ctx, 128]
 *   seq_lens, ret_heads as in rtp_index_topp
 *   sel_idx, sel_cnt    as written by rtp_index_topp for the same B, n_ret, max_ctx, block
 *   sel_mask   optional: the block masks rtp_index_topp wrote for the same sizes.  When it is
 *              not NULL the union of a split's blocks is read from it in one round of loads
 *              (sel_idx and sel_cnt are then not read and may be NULL); otherwise each
 *              head's ascending list is searched for the split's range.
 *   split_tokens  multiple of block; split_tokens / block <= 2048
 *   o_part     out fp32 [B, n_ret, n_split, 128], n_split = ceil(max_ctx / split_tokens)
 *   lse_part   out fp32 [B, n_ret, n_split]
 *   kv_slot, n_full  KV placement (see "KV placement" below); NULL: k_cache and v_cache
 *              hold every KV head ([B, Hkv, max_ctx, 128]).  A KV group with retrieval heads
 *              must be in the full caches (kv_slot[g] >= 0).
 */
rtp_status rtp_sparse_attn_split(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seq_lens, const int* ret_heads,
                                 const int* sel_idx, const int* sel_cnt, const unsigned char* sel_mask,
                                 int B, int Hq, int Hkv, int n_ret, int max_ctx, int block,
                                 int split_tokens, float* o_part, float* lse_part,
                                 const int* kv_slot, int n_full, void* stream);

/*
 * Cross-split log-sum-exp reduce (Strikes-Back architecture paragraph):
 *   L = log sum_c exp(lse_part[b, i, c]);  out[b, heads[i]] = sum_c exp(lse_c - L) o_part[b, i, c]
 * Splits with lse = -inf carry weight 0; a row whose splits are all empty is written 0.
 *
 *   o_part    fp32 [B, n_heads, n_split, 128]
 *   lse_part  fp32 [B, n_heads, n_split]
 *   heads     int32 [n_heads]   query-head id of partial row i
 *   out       out fp32 [B, Hq, 128]; only rows heads[] are written
 */
rtp_status rtp_split_reduce(const float* o_part, const float* lse_part, const int* heads,
                            int B, int Hq, int n_heads, int n_split, float* out, void* stream);

/* Bytes of workspace rtp_local_window_attn needs (0 if a size is invalid). */
size_t rtp_local_window_workspace_size(int B, int Hq, int Hkv, int n_loc, int max_ctx,
                                       int window, int sinks);

/*
 * Local heads: exact attention over attention sinks + a sliding window
 * (Review, Adaptive sparse attention: local heads keep a window and sinks; Review,
 * Experiments: sink 4, window 8192).
 *
 * For each sequence b and local head hq = loc_heads[i] (KV head g = hq / (Hq/Hkv)):
 *   T = [0, min(sinks, N)) union [max(0, N - window), N)   (no token counted twice)
 *   out[b, hq] = sum_{n in T} softmax_n(q[b,hq] . K[b,g,n] / sqrt(128)) V[b,g,n]
 * The window is split across workgroups (one per KV group and split, serving every
 * local head of the group) that write partials to the workspace; a second kernel on
 * the same stream merges them with the log-sum-exp rule.
 *
 *   q, k_cache, v_cache, seq_lens as in rtp_sparse_attn_split
 *   loc_heads int32 [n_loc]  query-head ids of the local heads, ascending
 *   window >= 0, sinks >= 0, window + sinks >= 1
 *   out       out fp32 [B, Hq, 128]; only rows loc_heads[] are written
 *   workspace >= rtp_local_window_workspace_size(B, Hq, Hkv, n_loc, max_ctx, window, sinks)
 *             bytes,
 *             zero-filled before first use
 *   kv_slot, n_full, k_ring, v_ring, n_ring  KV placement (above); NULL kv_slot: every group
 *             in k_cache / v_cache ([B, Hkv, max_ctx, 128]).  A ring group attends to its
 *             rows [0, min(N, sinks + window)): the same token set T.
 */
rtp_status rtp_local_window_attn(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seq_lens, const int* loc_heads,
                                 int B, int Hq, int Hkv, int n_loc, int max_ctx,
                                 int window, int sinks, float* out,
                                 void* workspace, size_t ws_bytes, const int* kv_slot, int n_full,
                                 const void* k_ring, const void* v_ring, int n_ring, void* stream);

/*
 * Decode-side cache maintenance, the step before the path: stores the decode token of
 * every sequence b at row pos = seq_lens[b] - 1 (the token is the last of the N_b tokens
 * the step attends to) (Review, Adaptive sparse attention equation, the key side of
 * s_h(m, n); Review, Method overview: retrieval heads keep the full KV cache):
 *   k_cache[b, g, pos] = k_new[b, g],  v_cache[b, g, pos] = v_new[b, g]   for every KV head g
 *   k_idx[b, r, pos, i] = bf16(sum_d W^K[r, i, d] k_pre[b, g_r, d])        for every retrieval
 *       head r (g_r = ret_heads[r] / (Hq / Hkv)) and i < 16: the exact sum of the 128
 *       products rounded once to nearest-even (an exact zero gives +0; a non-finite input
 *       gives the IEEE result of an fp64 sum: NaN or infinity)
 *
 *   k_new, v_new  bf16 [B, Hkv, 128]   the token's key (as the attention reads it) and value
 *   k_pre         bf16 [B, Hkv, 128]   the token's pre-RoPE key (the index projection's input)
 *   w_k           bf16 [n_ret, 16, 128] W^K of each retrieval head
 *   seq_lens      int32 [B]            N_b including the token, 1 <= N_b <= max_ctx
 *   k_cache, v_cache, k_idx            the caches of rtp_index_topp / rtp_sparse_attn_split;
 *                                      only row pos of each is written
 *   kv_slot, n_full, k_ring, v_ring, n_ring, sinks, window  KV placement (above): a ring
 *                                      group's token goes to its ring row; NULL kv_slot: every
 *                                      group in k_cache / v_cache ([B, Hkv, max_ctx, 128])
 * k_pre, w_k, ret_heads and k_idx may be NULL when n_ret == 0.  Device pointers 16-byte
 * aligned (k_idx 2-byte).
 */
rtp_status rtp_cache_append(const void* k_new, const void* v_new, const void* k_pre, const void* w_k,
                            const int* seq_lens, const int* ret_heads, int B, int Hq, int Hkv, int n_ret,
                            int max_ctx, void* k_cache, void* v_cache, void* k_idx, const int* kv_slot,
                            int n_full, void* k_ring, void* v_ring, int n_ring, int sinks, int window,
                            void* stream);

/*
 * The decode step's attention in one launch: rtp_sparse_attn_split's partials for the
 * retrieval heads (Strikes-Back method item 2 and architecture paragraph, Kernel 2) and
 * the local heads' window + sink partials (Review, Adaptive sparse attention: local heads
 * keep a window and sinks; the same token set T as rtp_local_window_attn) written to
 * ws_local, computed by the workgroups of one grid: the split attention's first (KV groups
 * heaviest first), the local heads' after them, so these fill the compute units the split
 * attention's last workgroups leave idle.  rtp_decode_merge turns both into outputs.
 *
 *   every argument as in rtp_sparse_attn_split (retrieval heads; NULL and ignored when
 *   n_ret == 0) and rtp_local_window_attn (local heads; ignored when n_loc == 0); ws_local
 *   holds the local partials (>= rtp_local_window_workspace_size bytes, 256-byte aligned)
 */
rtp_status rtp_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int* seq_lens,
                           const int* ret_heads, const int* sel_idx, const int* sel_cnt,
                           const unsigned char* sel_mask, const int* loc_heads, int B, int Hq, int Hkv,
                           int n_ret, int n_loc, int max_ctx, int block, int split_tokens, int window,
                           int sinks, float* o_part, float* lse_part, void* ws_local, size_t ws_local_bytes,
                           const int* kv_slot, int n_full, const void* k_ring, const void* v_ring, int n_ring,
                           void* stream);

/*
 * The decode step's merge in one launch (Strikes-Back architecture paragraph, the
 * cross-split reduce): out[b, ret_heads[i]] from the retrieval heads' split partials as
 * rtp_split_reduce computes it, and out[b, loc_heads[i]] from the local heads' window
 * partials rtp_decode_attn left in ws_local, with the same log-sum-exp rule.
 *
 *   o_part, lse_part  as written by rtp_decode_attn (n_split = ceil(max_ctx / split_tokens))
 *   ws_local          the local workspace of rtp_decode_attn (same sizes)
 *   out               out fp32 [B, Hq, 128]; rows ret_heads[] and loc_heads[] are written
 */
rtp_status rtp_decode_merge(const float* o_part, const float* lse_part, const int* ret_heads,
                            const int* loc_heads, int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx,
                            int split_tokens, int window, int sinks, const void* ws_local,
                            size_t ws_local_bytes, float* out, void* stream);

/*
 * One decode step in one host call, three launches (Strikes-Back architecture paragraph:
 * Kernel 1, Kernel 2 and the reduce; Review, Adaptive sparse attention: local heads):
 * rtp_index_topp (or rtp_index_topk), rtp_decode_attn and rtp_decode_merge for the same
 * arguments, on `stream`.  When side_stream, ev_fork and ev_join are given, there are
 * retrieval and local heads, and the local heads' K/V bytes (B * Hkv * min(window + sinks,
 * max_ctx) * 512) are at least 64 MiB and half the index keys' (B * n_ret * max_ctx * 32), the local
 * heads' part of rtp_decode_attn goes to side_stream instead (forked from `stream` by
 * recording ev_fork and waiting for it; joined by recording ev_join there and making
 * `stream` wait for it before the merge), so it overlaps the index kernel; the caller owns
 * the streams and the events (hipEvent_t as void*, created without timing).  The outputs
 * equal those of the separate calls rtp_index_topp, rtp_sparse_attn_split,
 * rtp_split_reduce and rtp_local_window_attn either way.  Every argument is checked before
 * anything is enqueued; after that it returns the first failing call's status.
 *
 *   k_tokens           0: the top-p rule with top_p (rtp_index_topp); > 0: the static top-k
 *                      rule with this budget (rtp_index_topk; top_p may then be NULL)
 *   o_part, lse_part   split partials as in rtp_sparse_attn_split (n_split =
 *                      ceil(max_ctx / split_tokens))
 *   ws_index           workspace of rtp_index_topp; ws_local of rtp_local_window_attn
 *   kv_slot, n_full, k_ring, v_ring, n_ring   KV placement (above), passed to the split
 *                      attention and the local heads
 *   every other argument as in the four calls
 */
rtp_status rtp_decode_step(const void* q_pre, const void* w_q, const void* k_idx, const void* q,
                           const void* k_cache, const void* v_cache, const int* seq_lens,
                           const int* ret_heads, const int* loc_heads, const float* top_p, int k_tokens,
                           int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx, int block,
                           int split_tokens, int window, int sinks,
                           int* sel_idx, int* sel_cnt, unsigned char* sel_mask,
                           float* o_part, float* lse_part, float* out,
                           void* ws_index, size_t ws_index_bytes, void* ws_local, size_t ws_local_bytes,
                           const int* kv_slot, int n_full, const void* k_ring, const void* v_ring, int n_ring,
                           void* stream, void* side_stream, void* ev_fork, void* ev_join);

/*
 * rtp_decode_step for callers that cannot allocate or pass workspaces (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same step with
 * the same kernels and arguments, except that the index workspace, the local heads'
 * workspace and the split partials (o_part, lse_part) live in a fixed array in the
 * library's device memory (rtp_decode_step_noalloc_limit() bytes on each GPU it runs on,
 * held until the process ends): at most 16 MiB of index workspace
 * (rtp_index_topp_workspace_size), 8 MiB of local workspace
 * (rtp_local_window_workspace_size) and 8 MiB of partials (B * n_ret * n_split * 516
 * bytes, rounded up), else RTP_ESCRATCH and nothing is enqueued.  It calls no allocating
 * routine.  The array's device address is looked up once per device (with that device
 * current); `stream` must belong to the current device.  The index part is cleared with a
 * fill kernel on `stream` at the first call on a device and whenever ceil(max_ctx / block)
 * changes; it keeps its per-head state between calls otherwise.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialized by the caller.  It runs on `stream` alone.  The index workspace's status words
 * are not reported by this entry point (a head whose wait ran out still selects every
 * block).  Outputs sel_idx, sel_cnt, sel_mask and out as in rtp_decode_step.
 */
size_t rtp_decode_step_noalloc_limit(void);
rtp_status rtp_decode_step_noalloc(const void* q_pre, const void* w_q, const void* k_idx, const void* q,
                                   const void* k_cache, const void* v_cache, const int* seq_lens,
                                   const int* ret_heads, const int* loc_heads, const float* top_p, int k_tokens,
                                   int B, int Hq, int Hkv, int n_ret, int n_loc, int max_ctx, int block,
                                   int split_tokens, int window, int sinks,
                                   int* sel_idx, int* sel_cnt, unsigned char* sel_mask, float* out,
                                   const int* kv_slot, int n_full, const void* k_ring, const void* v_ring,
                                   int n_ring, void* stream);

/*
 * Ring fill after a prefill (KV placement above): for every ring group (kv_slot[g] < 0),
 * ring row r of sequence b receives the K and V rows of the position it holds once the
 * prompt's N = seq_lens[b] tokens are in: r < S: position r (if r < N); r = S + j: the
 * latest position p < N with p >= max(S, N - W) and (p - S) mod W = j.  Rows no
 * position maps to are left untouched; full groups are skipped.
 *
 *   k, v           bf16 [B, Hkv, max_ctx, 128]  the prompt's keys and values
 *   kv_slot        int32 [Hkv] (device), slots in range (not checked)
 *   k_ring, v_ring bf16 [B, n_ring, sinks + window, 128]
 * n_ring == 0 is a no-op.  Device pointers 16-byte aligned.
 */
rtp_status rtp_ring_fill(const void* k, const void* v, const int* seq_lens, const int* kv_slot, int B, int Hkv,
                         int max_ctx, void* k_ring, void* v_ring, int n_ring, int sinks, int window,
                         void* stream);

/*
 * Prefill attention over whole prompts (Review, Adaptive sparse attention: local heads
 * apply the sliding window + sink rule in prefill as in decode; retrieval heads run full
 * dense attention; Review, Efficiency & ultra-long robustness: the prefill sparsity is
 * fixed in advance).  Causal: the query at prompt position i of query head h attends to
 *   retrieval head (h in ret_heads):  every position 0..i;
 *   local head:                       [0, min(S, i + 1)) union [max(0, i + 1 - W), i + 1).
 * out[b, h, i] = softmax(q_i K^T / sqrt(128)) V over that set, for i < seq_lens[b].
 *
 *   q          bf16 [B, Hq, max_ctx, 128]   row i = the query at position i
 *   k, v       bf16 [B, Hkv, max_ctx, 128]  the prompt's keys and values (e.g. the full caches);
 *                                           query head h uses KV head h / (Hq / Hkv)
 *   seq_lens   int32 [B]: prompt lengths, 1 <= seq_lens[b] <= max_ctx (device values, not
 *              checked); rows at or past seq_lens[b] are neither read nor written
 *   ret_heads  int32 [n_ret] retrieval query heads, distinct (NULL when n_ret == 0)
 *   window, sinks  W >= 0, S >= 0, W + S >= 1 (ignored when every head is a retrieval head)
 *   out        fp32 [B, Hq, max_ctx, 128]
 * Precision: q.k products exact, fp32 accumulation; probabilities and V enter the PV
 * product as fp16 (V values outside fp16's normal range, |v| < 2^-14 or > 65504, lose
 * precision or saturate).  Device pointers 16-byte aligned.
 */
rtp_status rtp_prefill_attn(const void* q, const void* k, const void* v, const int* seq_lens,
                            const int* ret_heads, int B, int Hq, int Hkv, int n_ret, int max_ctx,
                            int window, int sinks, float* out, void* stream);

/*
 * The prompt's index keys (Review, Adaptive sparse attention equation, the key side of
 * s_h(m, n)): k_idx[b, r, n] = bf16(W^K_r k^pre[b, g, n]) for n < seq_lens[b], every
 * retrieval head r (g its KV head), each the exact sum of the 128 products rounded once
 * to bf16, nearest-even, as rtp_cache_append does for one decode token.
 *
 *   k_pre  bf16 [B, Hkv, max_ctx, 128]   pre-RoPE keys
 *   w_k    bf16 [n_ret, 16, 128]
 *   k_idx  bf16 [B, n_ret, max_ctx, 16]  rows at or past seq_lens[b] untouched
 * n_ret == 0 is a no-op.  k_pre, w_k 16-byte aligned; k_idx 2-byte aligned.
 */
rtp_status rtp_prefill_index_keys(const void* k_pre, const void* w_k, const int* seq_lens,
                                  const int* ret_heads, int B, int Hq, int Hkv, int n_ret, int max_ctx,
                                  void* k_idx, void* stream);

/*
 * Calibration probe (not part of the decode path): reads `bytes` of device memory at
 * `src` once with 16-byte loads (non-temporal when `nontemporal` != 0, as the path's
 * streams use; else ordinary cached loads) over a grid-stride loop of n_workgroups
 * 256-thread workgroups, and writes one folded word per workgroup to sink[n_workgroups]
 * (so no load is dropped).  Timing it gives the read-only streaming rate the HBM-bound
 * kernels are compared with.  bytes a multiple of 16, src 16-byte aligned, 1 <=
 * n_workgroups <= 65535; else RTP_EINVAL.
 */
rtp_status rtp_stream_read(const void* src, size_t bytes, unsigned int* sink, int n_workgroups, int nontemporal,
                           void* stream);

/*
 * Calibration probe (not part of the path): n_workgroups 256-thread workgroups, each wave
 * issuing iters x 4 back-to-back v_mfma_f32_32x32x16_bf16 (32768 flops each) on four
 * independent accumulators, so timing it gives the bf16 MFMA rate the prefill kernel is
 * compared with (flops = n_workgroups * 16 * iters * 32768).  ops: device bf16 [2][64][8],
 * 16-byte aligned: lane l's eight A values, then its eight B values, the same in every
 * wave (the rate depends on the operands' bit patterns, so pass data like the workload's).
 * out[n_workgroups * 256] (device fp32): each thread's sum of its 64 accumulator elements
 * (4 x iters x the lane's 16 elements of A B in the MFMA's output layout).
 * 1 <= n_workgroups <= 65535, 1 <= iters <= 16384; else RTP_EINVAL.
 */
rtp_status rtp_mfma_rate(const void* ops, float* out, int n_workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H_ */
