/*
 * mla.h -- C ABI of the chunk-causal multi-head latent attention library
 * (libmla_hip.so, HIP kernels for AMD gfx950 / MI355X).
 *
 * What is computed.  VideoMLA (arXiv abstract on the mlsanity.com paper page;
 * atlas.scime.ai summary, "Approach") replaces per-head keys and values with
 * one low-rank content latent shared by all heads plus one head-shared,
 * decoupled 3D-RoPE positional key.  Each cached token therefore keeps the
 * row [c || k_R] of d_c + d_r scalars (224 at d_c = 192, d_r = 32, against
 * 3072 for 12 heads x 128 of dense K and V; atlas summary, "Key results").
 * Scores and up-projections follow multi-head latent attention as introduced
 * by DeepSeek-V2 (listed under "Builds on" on both VideoMLA pages):
 *
 *   append   c = W_DKV x,  k_R = RoPE3D(t,h,w) (W_KR x),  row = bf16([c || k_R])
 *   attend   s(i,h,j) = scale * ( q_h . (W_UK[h] c_j) + RoPE3D(p_i) q_r,h . k_R,j )
 *            O(i,h)   = sum_j softmax_j(s) W_UV[h] c_j
 * for a chunk of queries that sees every cached chunk and itself
 * (chunk-causal, bidirectional inside the chunk: atlas summary, first
 * paragraph).  The library evaluates attention in the absorbed form:
 *   q~ = [scale*log2(e) * W_UK[h]^T q_h || scale*log2(e) * RoPE3D(p_i) q_r,h]
 *   L  = softmax2(q~ . [c || k_R]) c      (fp32, over all visible keys)
 *   O  = W_UV[h] L
 * which is the same function up to rounding.
 *
 * Conventions for every entry point.
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never allocates, frees or retains them beyond the enqueued work.
 *   - Tensors are dense row-major with the shapes given, 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously; nothing here synchronizes the device unless
 *     the environment variable MLA_SYNC_CHECK=1 is set, in which case each
 *     launch is followed by a stream synchronize and device faults are
 *     reported as MLA_ERR_HIP.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is enqueued and a negative mla_status is returned.
 *     mla_last_error() gives a human-readable reason (thread-local).
 *   - The library keeps no global mutable state; calls are thread-safe.
 *     Calls that share a workspace must be ordered on one stream.
 *   - MLA_ATTEND_HEADROOM (read at each call; default 32, range 0..64) bounds
 *     the single-pass softmax of every bf16 attention kernel.  A key segment's
 *     reference maximum is its first 32-key block's; if, for some row, the
 *     running sum of p = 2^(s - m) over the keys one lane holds (half of the
 *     segment's keys) exceeds 2^headroom, or an accumulator is not finite, the
 *     segment is redone as an exact two-pass softmax.  Since every p <= that
 *     sum, no score then exceeds the reference maximum by more than headroom
 *     log2 units.  The rule is conservative (many keys near the maximum also
 *     trigger it once headroom < log2(keys per lane)); it changes rounding
 *     only, never the result beyond it.  Tests lower it to exercise the
 *     two-pass path.
 *   - dtype MLA_BF16 means every floating-point input of the call is bfloat16;
 *     MLA_F32 means every one is float32.  Positions are always int32.
 *
 * Weight layouts ("out x in", as in DeepSeek-V2's W^{DKV}, W^{KR}, W^{UK},
 * W^{UV}):
 *   w_dkv [d_c, d_model]   w_kr [d_r, d_model]
 *   w_uk  [H, d_h, d_c]    w_uv [H, d_h, d_c]
 * Cache layout: cache[b][slot][0 .. d_c)      = c  of the token in that slot
 *               cache[b][slot][d_c .. d_c+d_r) = k_R (already rotated)
 * i.e. [B, capacity, d_c + d_r], 2*(d_c+d_r) bytes per slot in bf16.
 *
 * 3D-RoPE reading (the pages name 3D-RoPE but give no formula): the d_r
 * vector is split into contiguous blocks of widths rope_t, rope_h, rope_w
 * (even, summing to d_r); inside a block of width d_a the adjacent pair
 * (2i, 2i+1) is rotated by angle p_a * rope_theta^(-2i/d_a), with
 * p = (t, h, w) the token's latent frame index, row and column.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size, out-of-range offset   */
  MLA_ERR_UNSUPPORTED = -2,  /* shape or dtype outside what the kernels are built for     */
  MLA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the required size       */
  MLA_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed                */
} mla_status;

typedef enum mla_dtype { MLA_BF16 = 0, MLA_F32 = 1 } mla_dtype;

/* Problem dimensions shared by all calls.  Supported: head_dim = 128,
 * d_c in {64, 128, 192, 256}, d_r = 32, rope_t + rope_h + rope_w = d_r with
 * each even, batch >= 1, n_heads >= 1, rope_theta > 0.
 * Wan2.1-1.3B shape: {1, 12, 128, 192, 32, 8, 12, 12, 1e4}. */
typedef struct mla_dims {
  int32_t batch;
  int32_t n_heads;
  int32_t head_dim;
  int32_t d_c;
  int32_t d_r;
  int32_t rope_t, rope_h, rope_w;
  double rope_theta;
} mla_dims;

/* Cache append (latent down-projection + rotated positional key).
 *   x        device [B, n_new, d_model]   hidden states of the new tokens
 *   w_dkv    device [d_c, d_model]        latent down-projection
 *   w_kr     device [d_r, d_model]        positional-key projection
 *   pos_thw  device int32 [n_new, 3]      (t, h, w) of each new token (shared by the batch)
 *   cache    device [B, cache_capacity, d_c + d_r]; slots write_offset ..
 *            write_offset + n_new - 1 of every sample are overwritten, all
 *            other slots are untouched.
 * Each output value is accumulated in fp32 from the dtype inputs, rotated in
 * fp32 with fp64-evaluated angles, and rounded once (to nearest even when the
 * dtype is bf16).  Requires d_model % 64 == 0 (bf16), n_new >= 0,
 * 0 <= write_offset, write_offset + n_new <= cache_capacity.  n_new == 0 is a
 * no-op returning MLA_OK. */
int32_t mla_cache_append(const mla_dims* dims, int32_t dtype,
                         const void* x, int32_t d_model, int32_t n_new,
                         const void* w_dkv, const void* w_kr,
                         const int32_t* pos_thw,
                         void* cache, int32_t cache_capacity, int32_t write_offset,
                         void* stream);

/* Bytes of device workspace mla_chunk_attend (and its three steps) needs for
 * these sizes; negative mla_status on invalid arguments. */
int64_t mla_chunk_attend_workspace_bytes(const mla_dims* dims, int32_t dtype,
                                         int32_t n_q, int32_t n_k);

/* One chunk step: absorb, attend, up-project (the three calls below, in order).
 *   q        device [B, n_q, H, d_h]     content queries of the current chunk
 *   q_r      device [B, n_q, H, d_r]     positional queries (rotated here)
 *   q_pos    device int32 [n_q, 3]       (t, h, w) of each query token
 *   w_uk, w_uv device [H, d_h, d_c]
 *   cache    device [B, cache_capacity, d_c + d_r]; keys are slots 0 .. n_k-1
 *            (all cached chunks plus the current chunk, already appended)
 *   softmax_scale  the score scale (e.g. 1/sqrt(d_h + d_r))
 *   out      device [B, n_q, H, d_h] of out_dtype
 *   workspace device, at least mla_chunk_attend_workspace_bytes(...) bytes;
 *            its contents on entry are irrelevant and on exit unspecified.
 * Requires 1 <= n_q <= n_k <= cache_capacity and, for bf16, n_k * (d_c + d_r) * 2 < 2^32
 * (one sample's visible keys below 4 GiB; MLA_ERR_UNSUPPORTED otherwise). */
int32_t mla_chunk_attend(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype,
                         const void* q, const void* q_r, const int32_t* q_pos, int32_t n_q,
                         const void* w_uk, const void* w_uv,
                         const void* cache, int32_t cache_capacity, int32_t n_k,
                         float softmax_scale, void* out,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* mla_chunk_attend without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and validation
 * as mla_chunk_attend, minus the workspace: the library's own static device
 * array of MLA_NOALLOC_SCRATCH_BYTES per GPU serves instead (held from the
 * first call on a device until the process ends).  Sizes whose workspace
 * (mla_chunk_attend_workspace_bytes) exceeds it return MLA_ERR_WORKSPACE,
 * before anything is enqueued.  Allocates nothing, on the host or the device.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or threads without ordering) race and must be
 * serialized by the caller. */
#define MLA_NOALLOC_SCRATCH_BYTES (128ll << 20)
int32_t mla_chunk_attend_noalloc(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype,
                                 const void* q, const void* q_r, const int32_t* q_pos, int32_t n_q,
                                 const void* w_uk, const void* w_uv,
                                 const void* cache, int32_t cache_capacity, int32_t n_k,
                                 float softmax_scale, void* out, void* stream);

/* Chunk-causal visibility for a call whose queries span several chunks (the
 * training / teacher-forcing form; VideoMLA atlas.scime.ai summary, first
 * paragraph: causal across chunks, bidirectional inside a chunk).  Query i
 * of the call is token q_start + i of the key sequence; with chunk length C
 * it sees keys [0, min(n_k, (floor((q_start + i) / C) + 1) * C)).
 * Requires C >= 1, q_start >= 0 and q_start + n_q <= n_k.  Tiles that no
 * query of a 256-row block can see are skipped. */
typedef struct mla_causal {
  int32_t q_start;
  int32_t chunk_len;
} mla_causal;

/* mla_chunk_attend with chunk-causal visibility (see mla_causal; `causal`
 * is a host pointer read during the call).  When n_k is a multiple of n_q,
 * q_start = n_k - n_q and chunk_len = n_q let every query see all n_k keys,
 * as mla_chunk_attend does. */
int32_t mla_chunk_attend_causal(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype,
                                const void* q, const void* q_r, const int32_t* q_pos, int32_t n_q,
                                const void* w_uk, const void* w_uv,
                                const void* cache, int32_t cache_capacity, int32_t n_k,
                                const mla_causal* causal, float softmax_scale, void* out,
                                void* workspace, int64_t workspace_bytes, void* stream);

/* Step 1 of mla_chunk_attend: writes the absorbed, pre-scaled queries q~
 * (the content part W_UK[h]^T q_h and the rotated positional part, both
 * multiplied by softmax_scale*log2(e), rounded once to the dtype) into the
 * workspace.  Arguments as for mla_chunk_attend. */
int32_t mla_query_absorb(const mla_dims* dims, int32_t dtype,
                         const void* q, const void* q_r, const int32_t* q_pos, int32_t n_q,
                         const void* w_uk, float softmax_scale, int32_t n_k,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* Step 2: fused score / online-softmax / P.c over all n_k keys for every
 * (batch, query, head) row, leaving fp32 partial softmax states in the
 * workspace.  Requires step 1 to have been enqueued with the same sizes. */
int32_t mla_latent_attend(const mla_dims* dims, int32_t dtype,
                          const void* cache, int32_t cache_capacity, int32_t n_q, int32_t n_k,
                          void* workspace, int64_t workspace_bytes, void* stream);

/* Step 2 with chunk-causal visibility (see mla_causal). */
int32_t mla_latent_attend_causal(const mla_dims* dims, int32_t dtype,
                                 const void* cache, int32_t cache_capacity, int32_t n_q, int32_t n_k,
                                 const mla_causal* causal,
                                 void* workspace, int64_t workspace_bytes, void* stream);

/* Step 3: merges the partial softmax states of each row into L (fp32) and
 * writes out = W_UV[h] L in out_dtype.  Requires steps 1 and 2. */
int32_t mla_value_upproj(const mla_dims* dims, int32_t dtype, int32_t out_dtype,
                         int32_t n_q, int32_t n_k, const void* w_uv, void* out,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* Standard multi-head attention over per-head keys and values: the dense
 * K/V cache the latent cache replaces (2 * H * d_h values per token against
 * d_c + d_r; VideoMLA atlas.scime.ai summary, "Key results"), provided as
 * the comparison point for the latent path.  For every (b, i, h):
 *   out[b,i,h,:] = sum_j softmax_j(softmax_scale * q[b,i,h,:] . k[b,j,h,:]) v[b,j,h,:]
 * over keys j = 0 .. n_k-1 (all visible: one chunk of queries that sees every
 * cached chunk and itself).  Positional encoding, if any, is already applied
 * to q and k.
 *   q    device bf16 [B, n_q, H, head_dim]
 *   k, v device bf16 [B, cache_capacity, H, head_dim]; slots 0 .. n_k-1 are read
 *   out  device [B, n_q, H, head_dim] of out_dtype (MLA_BF16 or MLA_F32)
 *   workspace device, at least mla_mha_attend_workspace_bytes(...) bytes.
 * Scores and P.V use bf16 MFMA with fp32 accumulation; the softmax is fp32
 * in base 2, with softmax_scale*log2(e) applied to the fp32 scores (q is
 * used as given, never rescaled and re-rounded); P is rounded to bf16.
 * Supported: head_dim = 128, 1 <= n_q <= n_k <= cache_capacity,
 * cache_capacity * n_heads * 256 < 2^32.  Errors as for mla_chunk_attend. */
int64_t mla_mha_attend_workspace_bytes(int32_t batch, int32_t n_heads, int32_t head_dim,
                                       int32_t n_q, int32_t n_k);
int32_t mla_mha_attend(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t out_dtype,
                       const void* q, int32_t n_q,
                       const void* k, const void* v, int32_t cache_capacity, int32_t n_k,
                       float softmax_scale, void* out,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* mla_chunk_attend in the non-absorbed form of multi-head latent attention
 * (DeepSeek-V2, listed under "Builds on" on both VideoMLA pages): per-head
 * keys and values are first materialised from the latent cache,
 *   K_h[j] = [W_UK[h] c_j || k_R,j]   (d_h + d_r),   V_h[j] = W_UV[h] c_j,
 * each rounded once to bf16 (fp32 accumulation), into the workspace; then
 * the attention of mla_mha_attend runs with queries [q_h || RoPE3D(p_i) q_r,h]
 * (the rotated part rounded once to bf16).
 * Same function as mla_chunk_attend up to rounding; it trades the absorbed
 * form's wider scores (d_c + d_r per key) for per-head K/V traffic.
 * Arguments as for mla_chunk_attend with in_dtype MLA_BF16.  Supported:
 * the mla_dims of mla_chunk_attend, n_k * n_heads * 320 < 2^32. */
int64_t mla_chunk_attend_expanded_workspace_bytes(const mla_dims* dims, int32_t n_q, int32_t n_k);
int32_t mla_chunk_attend_expanded(const mla_dims* dims, int32_t out_dtype,
                                  const void* q, const void* q_r, const int32_t* q_pos, int32_t n_q,
                                  const void* w_uk, const void* w_uv,
                                  const void* cache, int32_t cache_capacity, int32_t n_k,
                                  float softmax_scale, void* out,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* The faster of the two evaluation orders for a chunk step's shape, picked
 * from measured times on MI355X: MLA_FORM_EXPANDED (mla_chunk_attend_expanded)
 * when in_dtype is MLA_BF16 and n_q >= 1280 at d_c = 192 or n_q >= 448 at
 * d_c = 256 (and the per-head keys fit its limits); otherwise
 * MLA_FORM_ABSORBED (mla_chunk_attend).  At the 480P shape (d_c = 192, 4680
 * queries, 32760 keys) the non-absorbed form is about 13% faster; at d_c <=
 * 128 the absorbed form always is.  Negative mla_status on arguments
 * mla_chunk_attend would reject. */
enum { MLA_FORM_ABSORBED = 0, MLA_FORM_EXPANDED = 1 };
int32_t mla_chunk_attend_form(const mla_dims* dims, int32_t in_dtype, int32_t n_q, int32_t n_k);

/* Workspace bytes of mla_chunk_attend_auto: those of the form it picks. */
int64_t mla_chunk_attend_auto_workspace_bytes(const mla_dims* dims, int32_t in_dtype, int32_t n_q, int32_t n_k);

/* mla_chunk_attend through the form mla_chunk_attend_form picks (the same
 * function up to rounding); arguments and errors as for mla_chunk_attend,
 * with a workspace of at least mla_chunk_attend_auto_workspace_bytes. */
int32_t mla_chunk_attend_auto(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype,
                              const void* q, const void* q_r, const int32_t* q_pos, int32_t n_q,
                              const void* w_uk, const void* w_uv,
                              const void* cache, int32_t cache_capacity, int32_t n_k,
                              float softmax_scale, void* out,
                              void* workspace, int64_t workspace_bytes, void* stream);

/* Rolling latent cache for long rollouts (a fixed-size sliding window of
 * cached chunks: VideoMLA arXiv abstract), with `sink_chunks` leading
 * chunks kept for the whole rollout.  Host-side bookkeeping only; the cache
 * itself is the caller's [B, capacity, d_c + d_r] buffer.
 *   capacity = (sink_chunks + window_chunks + 1) * chunk_tokens
 * Chunk j (0-based) goes to chunk slot j while the ring fills; afterwards
 * chunk j >= sink_chunks goes to chunk slot
 * sink_chunks + (j - sink_chunks) mod (window_chunks + 1), the slot the
 * oldest window chunk leaves when chunk j-1 is committed.  The key range of
 * every step is slots [0, n_k), in slot order; attention does not depend on
 * key order and positional keys keep their absolute positions, so nothing
 * is moved.  All batch samples of one ring advance together; samples at
 * different rollout positions keep one ring each and are attended one call
 * per sample (batch 1) over their own slice of the cache, which starts at
 * element b * capacity * (d_c + d_r). */
typedef struct mla_ring {
  int32_t chunk_tokens;
  int32_t sink_chunks;
  int32_t window_chunks;
  int32_t capacity;      /* cache slots the ring needs */
  int64_t committed;     /* chunks committed so far = index of the current chunk */
} mla_ring;

/* Initialize an empty ring.  chunk_tokens >= 1, sink_chunks >= 0,
 * window_chunks >= 0.  The struct is plain data owned by the caller and the
 * library keeps no other state: saving it together with each sample's cache
 * slots [0, capacity) checkpoints a rollout, and restoring both resumes it
 * exactly (the next steps write the same slots and attend to the same keys). */
int32_t mla_ring_init(mla_ring* ring, int32_t chunk_tokens, int32_t sink_chunks, int32_t window_chunks);

/* Where the current chunk goes and which keys its steps attend to: append
 * its tokens with mla_cache_append(..., write_offset), then attend with
 * n_k keys (every cached chunk plus the current one).  Repeated denoising
 * steps of the same chunk overwrite the same slots. */
int32_t mla_ring_current(const mla_ring* ring, int32_t* write_offset, int32_t* n_k);

/* The current chunk's last denoising step is done: it joins the cache (the
 * oldest non-sink chunk leaves if the window is full). */
int32_t mla_ring_commit(mla_ring* ring);

/* Host array [sink_chunks + window_chunks + 1]: the chunk index held by each
 * chunk slot (the current chunk included), or -1 for an empty slot. */
int32_t mla_ring_slot_chunks(const mla_ring* ring, int64_t* chunk_of_slot);

/* Bytes of a latent cache of `capacity` slots for all B samples (one layer),
 * and of the dense per-head K and V cache it replaces (2 * H * d_h values
 * per token; VideoMLA atlas.scime.ai summary, "Key results": 224 against 3072
 * scalars per token at d_c = 192).  Negative mla_status on invalid
 * arguments. */
int64_t mla_cache_bytes(const mla_dims* dims, int32_t dtype, int32_t capacity);
int64_t mla_dense_kv_bytes(const mla_dims* dims, int32_t dtype, int32_t capacity);

/* Reason for the last failed mla_ring_* or byte-count call on this thread. */
const char* mla_ring_last_error(void);

/* Static description of a status code. */
const char* mla_status_string(int32_t status);

/* Reason for the last non-OK status returned on the calling thread. */
const char* mla_last_error(void);

/* Library version and the gfx target it was built for, e.g. "0.1.0 gfx950". */
const char* mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
