// C ABI of the latent-attention library: argument validation (host only,
// nothing is enqueued on error), workspace planning and kernel dispatch.
// Declarations and contracts: include/mla.h.
#include "mla.h"

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mla_common.h"
#include "mla_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

bool sync_check() {
  static const bool on = [] {
    const char* v = getenv("MLA_SYNC_CHECK");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

int32_t finish(hipError_t launched, hipStream_t s, const char* what) {
  if (launched != hipSuccess)
    return fail(MLA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(launched));
  if (sync_check()) {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: kernel failed: %s", what, hipGetErrorString(e));
  }
  return MLA_OK;
}

// Headroom (log2 units) of the single-pass attention: a key segment whose
// lane-wise running sum of p = 2^(s - m) exceeds 2^headroom (m = its
// first-block max; every p is at most that sum, so no score exceeds m by more)
// is redone in two exact passes, in every bf16 attention kernel.  32 by
// default; MLA_ATTEND_HEADROOM (read at every call) overrides it, so tests can
// set it small and exercise the two-pass path on ordinary inputs.
float attend_headroom() {
  const char* v = getenv("MLA_ATTEND_HEADROOM");
  const float x = v ? (float)atof(v) : 32.0f;
  return (x >= 0.f && x <= 64.f) ? x : 32.0f;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int32_t check_dims(const mla_dims* d) {
  if (d == nullptr) return fail(MLA_ERR_INVALID_ARG, "dims is null");
  if (d->batch < 1 || d->n_heads < 1) return fail(MLA_ERR_INVALID_ARG, "batch and n_heads must be >= 1");
  if (d->head_dim != 128) return fail(MLA_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", d->head_dim);
  if (d->d_c != 64 && d->d_c != 128 && d->d_c != 192 && d->d_c != 256)
    return fail(MLA_ERR_UNSUPPORTED, "d_c must be 64, 128, 192 or 256 (got %d)", d->d_c);
  if (d->d_r != 32) return fail(MLA_ERR_UNSUPPORTED, "d_r must be 32 (got %d)", d->d_r);
  if (d->rope_t < 0 || d->rope_h < 0 || d->rope_w < 0 || (d->rope_t | d->rope_h | d->rope_w) & 1 ||
      d->rope_t + d->rope_h + d->rope_w != d->d_r)
    return fail(MLA_ERR_UNSUPPORTED, "rope widths must be even and sum to d_r (got %d/%d/%d)",
                d->rope_t, d->rope_h, d->rope_w);
  if (!(d->rope_theta > 0.0)) return fail(MLA_ERR_INVALID_ARG, "rope_theta must be > 0");
  return MLA_OK;
}

int32_t check_dtype(int32_t dt, const char* name) {
  if (dt != MLA_BF16 && dt != MLA_F32) return fail(MLA_ERR_UNSUPPORTED, "%s must be MLA_BF16 or MLA_F32 (got %d)", name, dt);
  return MLA_OK;
}

int32_t check_ptr(const void* p, const char* name, uintptr_t align = 16) {
  if (p == nullptr) return fail(MLA_ERR_INVALID_ARG, "%s is null", name);
  if (!aligned(p, align)) return fail(MLA_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, (int)align);
  return MLA_OK;
}

mla::RopeSpec rope_of(const mla_dims* d) { return mla::RopeSpec{d->rope_t, d->rope_h, d->rope_w, d->rope_theta}; }

// Sizes shared by the chunk-attend steps; fills the plan on success.
int32_t check_attend_sizes(const mla_dims* d, int32_t dtype, int32_t n_q, int32_t n_k, mla::Plan* plan) {
  int32_t st = check_dims(d);
  if (st) return st;
  if ((st = check_dtype(dtype, "dtype"))) return st;
  if (n_q < 1) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 1 (got %d)", n_q);
  if (n_k < n_q) return fail(MLA_ERR_INVALID_ARG, "n_k (%d) must be >= n_q (%d): the current chunk is part of the keys", n_k, n_q);
  if ((int64_t)d->n_heads * n_q > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "n_heads * n_q too large");
  if ((int64_t)d->batch * ((int64_t)d->n_heads * n_q + 255) / 256 > (int64_t)1 << 24)
    return fail(MLA_ERR_UNSUPPORTED, "batch * rows too large");
  // the attention kernels address a sample's keys with 32-bit byte offsets
  if (dtype == MLA_BF16 && (int64_t)n_k * (d->d_c + d->d_r) * 2 >= (int64_t)1 << 32)
    return fail(MLA_ERR_UNSUPPORTED, "n_k (%d) too large: one sample's keys must stay below 4 GiB", n_k);
  *plan = mla::make_plan(d->batch, d->n_heads, n_q, n_k, d->d_c, d->d_r, dtype == MLA_F32);
  return MLA_OK;
}

int32_t check_workspace(const mla::Plan& p, const void* ws, int64_t bytes) {
  if (ws == nullptr) return fail(MLA_ERR_WORKSPACE, "workspace is null");
  if (!aligned(ws, 256)) return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < p.total)
    return fail(MLA_ERR_WORKSPACE, "workspace has %lld bytes, %lld needed", (long long)bytes, (long long)p.total);
  return MLA_OK;
}

int32_t do_absorb(const mla_dims* d, int32_t dtype, const mla::Plan& p, const void* q, const void* q_r,
                  const int32_t* q_pos, const void* w_uk, float scale, void* ws, hipStream_t s) {
  mla::AbsorbArgs a{};
  a.q = q; a.q_r = q_r; a.q_pos = q_pos; a.w_uk = w_uk;
  a.qscale = (float)((double)scale * mla::kLog2e);
  a.qt = (char*)ws + p.off_qt;
  a.rope = rope_of(d);
  hipError_t e = dtype == MLA_BF16 ? mla::launch_absorb_bf16(p, a, s) : mla::launch_absorb_f32(p, a, s);
  return finish(e, s, "mla_query_absorb");
}

// Chunk-causal limits of a call (nullptr: every query sees all n_k keys).
int32_t check_causal(const mla_causal* c, int32_t n_q, int32_t n_k) {
  if (c == nullptr) return fail(MLA_ERR_INVALID_ARG, "causal is null");
  if (c->chunk_len < 1) return fail(MLA_ERR_INVALID_ARG, "causal.chunk_len must be >= 1 (got %d)", c->chunk_len);
  if (c->q_start < 0 || (int64_t)c->q_start + n_q > n_k)
    return fail(MLA_ERR_INVALID_ARG, "causal.q_start %d + n_q %d must lie within n_k %d", c->q_start, n_q, n_k);
  if ((int64_t)n_k + c->chunk_len > (int64_t)INT32_MAX) return fail(MLA_ERR_UNSUPPORTED, "n_k + chunk_len too large");
  return MLA_OK;
}

mla::Visibility visibility(const mla::Plan& p, const mla_causal* causal) {
  return mla::Visibility{p.n_q, p.rows_b, causal ? causal->q_start : 0, causal ? causal->chunk_len : 0};
}

// The plan of a chunk-causal call: per-row-block units (same workspace size).
mla::Plan causal_plan(const mla_dims* d, int32_t dtype, const mla::Plan& p, const mla_causal* causal) {
  if (causal == nullptr) return p;
  const mla::Visibility vis = visibility(p, causal);
  return mla::make_plan(d->batch, d->n_heads, p.n_q, p.n_k, d->d_c, d->d_r, dtype == MLA_F32, &vis);
}

int32_t do_attend(const mla_dims* d, int32_t dtype, const mla::Plan& p, const void* cache, int32_t cap,
                  const mla_causal* causal, void* ws, hipStream_t s) {
  mla::AttendArgs a{};
  a.cache = cache;
  a.cache_bstride = (int64_t)cap * (d->d_c + d->d_r);
  a.workspace = ws;
  a.headroom = attend_headroom();
  a.vis = visibility(p, causal);
  hipError_t e = dtype == MLA_BF16 ? mla::launch_attend_bf16(p, a, s) : mla::launch_attend_f32(p, a, s);
  return finish(e, s, "mla_latent_attend");
}

int32_t do_upproj(int32_t dtype, int32_t out_dtype, const mla::Plan& p, const void* w_uv, void* out,
                  void* ws, hipStream_t s) {
  mla::UpprojArgs a{};
  a.w_uv = w_uv; a.out = out; a.out_f32 = out_dtype == MLA_F32; a.workspace = ws;
  hipError_t e = dtype == MLA_BF16 ? mla::launch_upproj_bf16(p, a, s) : mla::launch_upproj_f32(p, a, s);
  return finish(e, s, "mla_value_upproj");
}

}  // namespace

namespace {

int32_t latent_attend_impl(const mla_dims* dims, int32_t dtype, const void* cache, int32_t cache_capacity,
                           int32_t n_q, int32_t n_k, const mla_causal* causal, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, dtype, n_q, n_k, &p);
  if (st) return st;
  if ((st = check_ptr(cache, "cache"))) return st;
  if (n_k > cache_capacity) return fail(MLA_ERR_INVALID_ARG, "n_k (%d) exceeds cache_capacity (%d)", n_k, cache_capacity);
  if (causal && (st = check_causal(causal, n_q, n_k))) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes))) return st;
  return do_attend(dims, dtype, causal_plan(dims, dtype, p, causal), cache, cache_capacity, causal, workspace,
                   (hipStream_t)stream);
}

int32_t chunk_attend_impl(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype, const void* q,
                          const void* q_r, const int32_t* q_pos, int32_t n_q, const void* w_uk, const void* w_uv,
                          const void* cache, int32_t cache_capacity, int32_t n_k, const mla_causal* causal,
                          float softmax_scale, void* out, void* workspace, int64_t workspace_bytes, void* stream) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, in_dtype, n_q, n_k, &p);
  if (st) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_ptr(q, "q"))) return st;
  if ((st = check_ptr(q_r, "q_r"))) return st;
  if ((st = check_ptr(q_pos, "q_pos", 4))) return st;
  if ((st = check_ptr(w_uk, "w_uk"))) return st;
  if ((st = check_ptr(w_uv, "w_uv"))) return st;
  if ((st = check_ptr(cache, "cache"))) return st;
  if ((st = check_ptr(out, "out"))) return st;
  if (n_k > cache_capacity) return fail(MLA_ERR_INVALID_ARG, "n_k (%d) exceeds cache_capacity (%d)", n_k, cache_capacity);
  if (causal && (st = check_causal(causal, n_q, n_k))) return st;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if ((st = check_workspace(p, workspace, workspace_bytes))) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = do_absorb(dims, in_dtype, p, q, q_r, q_pos, w_uk, softmax_scale, workspace, s))) return st;
  if ((st = do_attend(dims, in_dtype, causal_plan(dims, in_dtype, p, causal), cache, cache_capacity, causal,
                      workspace, s)))
    return st;
  return do_upproj(in_dtype, out_dtype, p, w_uv, out, workspace, s);
}

// ---------------------------------------------------------------------------
// Standard attention over per-head K/V (dense baseline, non-absorbed form).
// ---------------------------------------------------------------------------
int32_t check_mha_sizes(int32_t batch, int32_t n_heads, int32_t n_q, int32_t n_k, int32_t dqk) {
  if (batch < 1 || n_heads < 1) return fail(MLA_ERR_INVALID_ARG, "batch and n_heads must be >= 1");
  if (n_heads > 4096) return fail(MLA_ERR_UNSUPPORTED, "n_heads must be <= 4096 (got %d)", n_heads);
  if (batch > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch must be <= 65535");
  if (n_q < 1) return fail(MLA_ERR_INVALID_ARG, "n_q must be >= 1 (got %d)", n_q);
  if (n_k < n_q) return fail(MLA_ERR_INVALID_ARG, "n_k (%d) must be >= n_q (%d): the current chunk is part of the keys", n_k, n_q);
  if ((int64_t)batch * n_heads * ((int64_t)n_q + 255) > (int64_t)1 << 30)
    return fail(MLA_ERR_UNSUPPORTED, "batch * n_heads * n_q too large");
  if ((int64_t)batch * n_k > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "batch * n_k too large");
  (void)dqk;
  return MLA_OK;
}

int32_t check_mha_capacity(int32_t n_heads, int32_t n_k, int32_t cap, int32_t dqk) {
  if (n_k > cap) return fail(MLA_ERR_INVALID_ARG, "n_k (%d) exceeds cache_capacity (%d)", n_k, cap);
  // key offsets inside one (batch, head) are 32-bit
  if ((int64_t)cap * n_heads * dqk * 2 >= (int64_t)1 << 32)
    return fail(MLA_ERR_UNSUPPORTED, "cache_capacity * n_heads too large (one sample's K must stay below 4 GiB)");
  return MLA_OK;
}

int32_t check_mha_workspace(const mla::MhaPlan& p, const void* ws, int64_t bytes) {
  if (ws == nullptr) return fail(MLA_ERR_WORKSPACE, "workspace is null");
  if (!aligned(ws, 256)) return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < p.total)
    return fail(MLA_ERR_WORKSPACE, "workspace has %lld bytes, %lld needed", (long long)bytes, (long long)p.total);
  return MLA_OK;
}

int32_t do_mha_attend(const mla::MhaPlan& p, const void* k, const void* v, int64_t cap, bool head_major, float scale,
                      int32_t out_dtype, void* out, void* ws, hipStream_t s, const char* what) {
  mla::MhaAttendArgs a{};
  a.k = k; a.v = v; a.cap = cap; a.head_major = head_major; a.headroom = attend_headroom();
  a.qscale = (float)((double)scale * mla::kLog2e);
  a.out = out; a.out_f32 = out_dtype == MLA_F32; a.workspace = ws;
  return finish(mla::launch_mha_attend(p, a, s), s, what);
}

}  // namespace

extern "C" {

int64_t mla_mha_attend_workspace_bytes(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t n_q, int32_t n_k) {
  if (head_dim != 128) return fail(MLA_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  int32_t st = check_mha_sizes(batch, n_heads, n_q, n_k, 128);
  if (st) return st;
  return mla::make_mha_plan(batch, n_heads, n_q, n_k, 128, false).total;
}

int32_t mla_mha_attend(int32_t batch, int32_t n_heads, int32_t head_dim, int32_t out_dtype, const void* q,
                       int32_t n_q, const void* k, const void* v, int32_t cache_capacity, int32_t n_k,
                       float softmax_scale, void* out, void* workspace, int64_t workspace_bytes, void* stream) {
  if (head_dim != 128) return fail(MLA_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  int32_t st = check_mha_sizes(batch, n_heads, n_q, n_k, 128);
  if (st) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_ptr(q, "q"))) return st;
  if ((st = check_ptr(k, "k"))) return st;
  if ((st = check_ptr(v, "v"))) return st;
  if ((st = check_ptr(out, "out"))) return st;
  if ((st = check_mha_capacity(n_heads, n_k, cache_capacity, 128))) return st;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const mla::MhaPlan p = mla::make_mha_plan(batch, n_heads, n_q, n_k, 128, false);
  if ((st = check_mha_workspace(p, workspace, workspace_bytes))) return st;
  hipStream_t s = (hipStream_t)stream;
  mla::MhaQueryArgs qa{};
  qa.q = q; qa.workspace = workspace;
  if ((st = finish(mla::launch_mha_prep_q(p, qa, s), s, "mla_mha_attend"))) return st;
  return do_mha_attend(p, k, v, cache_capacity, false, softmax_scale, out_dtype, out, workspace, s, "mla_mha_attend");
}

int64_t mla_chunk_attend_expanded_workspace_bytes(const mla_dims* dims, int32_t n_q, int32_t n_k) {
  int32_t st = check_dims(dims);
  if (st) return st;
  if ((st = check_mha_sizes(dims->batch, dims->n_heads, n_q, n_k, 160))) return st;
  return mla::make_mha_plan(dims->batch, dims->n_heads, n_q, n_k, 160, true).total;
}

int32_t mla_chunk_attend_expanded(const mla_dims* dims, int32_t out_dtype, const void* q, const void* q_r,
                                  const int32_t* q_pos, int32_t n_q, const void* w_uk, const void* w_uv,
                                  const void* cache, int32_t cache_capacity, int32_t n_k, float softmax_scale,
                                  void* out, void* workspace, int64_t workspace_bytes, void* stream) {
  int32_t st = check_dims(dims);
  if (st) return st;
  if ((st = check_mha_sizes(dims->batch, dims->n_heads, n_q, n_k, 160))) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_ptr(q, "q"))) return st;
  if ((st = check_ptr(q_r, "q_r"))) return st;
  if ((st = check_ptr(q_pos, "q_pos", 4))) return st;
  if ((st = check_ptr(w_uk, "w_uk"))) return st;
  if ((st = check_ptr(w_uv, "w_uv"))) return st;
  if ((st = check_ptr(cache, "cache"))) return st;
  if ((st = check_ptr(out, "out"))) return st;
  if (n_k > cache_capacity) return fail(MLA_ERR_INVALID_ARG, "n_k (%d) exceeds cache_capacity (%d)", n_k, cache_capacity);
  if ((st = check_mha_capacity(dims->n_heads, n_k, n_k, 160))) return st;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const mla::MhaPlan p = mla::make_mha_plan(dims->batch, dims->n_heads, n_q, n_k, 160, true);
  if ((st = check_mha_workspace(p, workspace, workspace_bytes))) return st;
  hipStream_t s = (hipStream_t)stream;
  mla::MhaQueryArgs qa{};
  qa.q = q; qa.q_r = q_r; qa.q_pos = q_pos; qa.rope = rope_of(dims);
  qa.workspace = workspace;
  if ((st = finish(mla::launch_mha_prep_q(p, qa, s), s, "mla_chunk_attend_expanded"))) return st;
  mla::MhaUpliftArgs ua{};
  ua.cache = cache; ua.cap = cache_capacity; ua.d_c = dims->d_c; ua.w_uk = w_uk; ua.w_uv = w_uv; ua.workspace = workspace;
  if ((st = finish(mla::launch_mha_uplift(p, ua, s), s, "mla_chunk_attend_expanded"))) return st;
  const char* ws = (const char*)workspace;
  return do_mha_attend(p, ws + p.off_k, ws + p.off_v, n_k, true, softmax_scale, out_dtype, out, workspace, s,
                       "mla_chunk_attend_expanded");
}

int32_t mla_cache_append(const mla_dims* dims, int32_t dtype, const void* x, int32_t d_model, int32_t n_new,
                         const void* w_dkv, const void* w_kr, const int32_t* pos_thw, void* cache,
                         int32_t cache_capacity, int32_t write_offset, void* stream) {
  int32_t st = check_dims(dims);
  if (st) return st;
  if ((st = check_dtype(dtype, "dtype"))) return st;
  if (n_new < 0) return fail(MLA_ERR_INVALID_ARG, "n_new must be >= 0");
  if (d_model < 1) return fail(MLA_ERR_INVALID_ARG, "d_model must be >= 1");
  if (dtype == MLA_BF16 && d_model % 64 != 0)
    return fail(MLA_ERR_UNSUPPORTED, "d_model must be a multiple of 64 for bf16 (got %d)", d_model);
  if (cache_capacity < 1 || write_offset < 0 || (int64_t)write_offset + n_new > cache_capacity)
    return fail(MLA_ERR_INVALID_ARG, "write_offset %d + n_new %d exceeds cache_capacity %d", write_offset, n_new,
                cache_capacity);
  if ((int64_t)dims->batch * n_new > (int64_t)1 << 30) return fail(MLA_ERR_UNSUPPORTED, "batch * n_new too large");
  if ((st = check_ptr(x, "x"))) return st;
  if ((st = check_ptr(w_dkv, "w_dkv"))) return st;
  if ((st = check_ptr(w_kr, "w_kr"))) return st;
  if ((st = check_ptr(pos_thw, "pos_thw", 4))) return st;
  if ((st = check_ptr(cache, "cache"))) return st;
  if (n_new == 0) return MLA_OK;
  mla::AppendArgs a{};
  a.batch = dims->batch; a.n_new = n_new; a.d_model = d_model; a.d_c = dims->d_c; a.d_r = dims->d_r;
  a.cap = cache_capacity; a.off = write_offset;
  a.x = x; a.w_dkv = w_dkv; a.w_kr = w_kr; a.pos = pos_thw; a.cache = cache;
  a.rope = rope_of(dims);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == MLA_BF16 ? mla::launch_append_bf16(a, s) : mla::launch_append_f32(a, s);
  return finish(e, s, "mla_cache_append");
}

int64_t mla_chunk_attend_workspace_bytes(const mla_dims* dims, int32_t dtype, int32_t n_q, int32_t n_k) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, dtype, n_q, n_k, &p);
  if (st) return st;
  return p.total;
}

int32_t mla_query_absorb(const mla_dims* dims, int32_t dtype, const void* q, const void* q_r,
                         const int32_t* q_pos, int32_t n_q, const void* w_uk, float softmax_scale, int32_t n_k,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, dtype, n_q, n_k, &p);
  if (st) return st;
  if ((st = check_ptr(q, "q"))) return st;
  if ((st = check_ptr(q_r, "q_r"))) return st;
  if ((st = check_ptr(q_pos, "q_pos", 4))) return st;
  if ((st = check_ptr(w_uk, "w_uk"))) return st;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if ((st = check_workspace(p, workspace, workspace_bytes))) return st;
  return do_absorb(dims, dtype, p, q, q_r, q_pos, w_uk, softmax_scale, workspace, (hipStream_t)stream);
}


int32_t mla_latent_attend(const mla_dims* dims, int32_t dtype, const void* cache, int32_t cache_capacity,
                          int32_t n_q, int32_t n_k, void* workspace, int64_t workspace_bytes, void* stream) {
  return latent_attend_impl(dims, dtype, cache, cache_capacity, n_q, n_k, nullptr, workspace, workspace_bytes,
                            stream);
}

int32_t mla_latent_attend_causal(const mla_dims* dims, int32_t dtype, const void* cache, int32_t cache_capacity,
                                 int32_t n_q, int32_t n_k, const mla_causal* causal, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
  if (causal == nullptr) return fail(MLA_ERR_INVALID_ARG, "causal is null");
  return latent_attend_impl(dims, dtype, cache, cache_capacity, n_q, n_k, causal, workspace, workspace_bytes,
                            stream);
}

int32_t mla_value_upproj(const mla_dims* dims, int32_t dtype, int32_t out_dtype, int32_t n_q, int32_t n_k,
                         const void* w_uv, void* out, void* workspace, int64_t workspace_bytes, void* stream) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, dtype, n_q, n_k, &p);
  if (st) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_ptr(w_uv, "w_uv"))) return st;
  if ((st = check_ptr(out, "out"))) return st;
  if ((st = check_workspace(p, workspace, workspace_bytes))) return st;
  return do_upproj(dtype, out_dtype, p, w_uv, out, workspace, (hipStream_t)stream);
}

int32_t mla_chunk_attend(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype, const void* q, const void* q_r,
                         const int32_t* q_pos, int32_t n_q, const void* w_uk, const void* w_uv, const void* cache,
                         int32_t cache_capacity, int32_t n_k, float softmax_scale, void* out, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  return chunk_attend_impl(dims, in_dtype, out_dtype, q, q_r, q_pos, n_q, w_uk, w_uv, cache, cache_capacity, n_k,
                           nullptr, softmax_scale, out, workspace, workspace_bytes, stream);
}

int32_t mla_chunk_attend_causal(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype, const void* q,
                                const void* q_r, const int32_t* q_pos, int32_t n_q, const void* w_uk,
                                const void* w_uv, const void* cache, int32_t cache_capacity, int32_t n_k,
                                const mla_causal* causal, float softmax_scale, void* out, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  if (causal == nullptr) return fail(MLA_ERR_INVALID_ARG, "causal is null");
  return chunk_attend_impl(dims, in_dtype, out_dtype, q, q_r, q_pos, n_q, w_uk, w_uv, cache, cache_capacity, n_k,
                           causal, softmax_scale, out, workspace, workspace_bytes, stream);
}

int32_t mla_chunk_attend_form(const mla_dims* dims, int32_t in_dtype, int32_t n_q, int32_t n_k) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, in_dtype, n_q, n_k, &p);
  if (st) return st;
  // Thresholds from timing both forms on MI355X (n_k = 32760; d_c 64-256):
  // the non-absorbed form wins at d_c = 192 from about 1280 queries per chunk
  // (absorbed 2% faster at 1152, 3% slower at 1280) and at d_c = 256 from
  // about 448 (level at 384, absorbed 8% slower at 448); at d_c <= 128 the
  // absorbed form always.
  const int32_t from = dims->d_c >= 256 ? 448 : dims->d_c >= 192 ? 1280 : INT32_MAX;
  if (in_dtype != MLA_BF16 || n_q < from) return MLA_FORM_ABSORBED;
  if (check_mha_sizes(dims->batch, dims->n_heads, n_q, n_k, 160) ||
      (int64_t)n_k * dims->n_heads * 160 * 2 >= (int64_t)1 << 32)
    return MLA_FORM_ABSORBED;
  return MLA_FORM_EXPANDED;
}

int64_t mla_chunk_attend_auto_workspace_bytes(const mla_dims* dims, int32_t in_dtype, int32_t n_q, int32_t n_k) {
  const int32_t form = mla_chunk_attend_form(dims, in_dtype, n_q, n_k);
  if (form < 0) return form;
  return form == MLA_FORM_EXPANDED ? mla_chunk_attend_expanded_workspace_bytes(dims, n_q, n_k)
                                   : mla_chunk_attend_workspace_bytes(dims, in_dtype, n_q, n_k);
}

int32_t mla_chunk_attend_auto(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype, const void* q,
                              const void* q_r, const int32_t* q_pos, int32_t n_q, const void* w_uk, const void* w_uv,
                              const void* cache, int32_t cache_capacity, int32_t n_k, float softmax_scale, void* out,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  const int32_t form = mla_chunk_attend_form(dims, in_dtype, n_q, n_k);
  if (form < 0) return form;
  if (form == MLA_FORM_EXPANDED)
    return mla_chunk_attend_expanded(dims, out_dtype, q, q_r, q_pos, n_q, w_uk, w_uv, cache, cache_capacity, n_k,
                                     softmax_scale, out, workspace, workspace_bytes, stream);
  return chunk_attend_impl(dims, in_dtype, out_dtype, q, q_r, q_pos, n_q, w_uk, w_uv, cache, cache_capacity, n_k,
                           nullptr, softmax_scale, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Chunk step with the library's own scratch (callers that cannot allocate).
//
// The workspace of mla_chunk_attend lives in a static device array of
// MLA_NOALLOC_SCRATCH_BYTES.  Its address on a device is taken once, with that
// device current, and kept per device; host code never uses the array's name
// as an address (on the host it is only a stand-in for the symbol).  Nothing
// in the workspace needs to start at zero: every kernel writes what it reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`.
int32_t scratch_for(hipStream_t stream, void** ptr) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MLA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_chunk_attend_noalloc(const mla_dims* dims, int32_t in_dtype, int32_t out_dtype, const void* q,
                                 const void* q_r, const int32_t* q_pos, int32_t n_q, const void* w_uk,
                                 const void* w_uv, const void* cache, int32_t cache_capacity, int32_t n_k,
                                 float softmax_scale, void* out, void* stream) {
  mla::Plan p;
  int32_t st = check_attend_sizes(dims, in_dtype, n_q, n_k, &p);
  if (st) return st;
  if (p.total > kScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "these sizes need %lld bytes of workspace; the no-allocation entry point has %lld",
                (long long)p.total, (long long)kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_for((hipStream_t)stream, &ws))) return st;
  return chunk_attend_impl(dims, in_dtype, out_dtype, q, q_r, q_pos, n_q, w_uk, w_uv, cache, cache_capacity, n_k,
                           nullptr, softmax_scale, out, ws, kScratchBytes, stream);
}

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_last_error; }

const char* mla_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
