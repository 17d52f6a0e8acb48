// Rolling latent cache: slot bookkeeping for long rollouts (host code).
//
// VideoMLA generates video chunk by chunk and, for long rollouts, keeps a
// fixed-size sliding window of cached chunks (arXiv abstract on the
// mlsanity.com paper page).  The ring here keeps `sink_chunks` leading chunks
// for the whole rollout plus the `window_chunks` most recent ones, and one
// chunk slot for the chunk being denoised.  Chunk j >= sink_chunks lives in
// chunk slot sink + (j - sink) mod (window + 1), so the slot the next chunk
// needs is exactly the one the oldest window chunk leaves on commit, and the
// state is the committed-chunk count alone.  Attention sees slots
// [0, n_k): once the window is full every slot is live and the keys are in
// slot order, not chunk order -- softmax does not depend on key order, and
// the positional keys carry their absolute positions from the append, so
// nothing is ever moved.
#include <stdio.h>
#include <stdarg.h>

#include "mla.h"

namespace {
thread_local char g_ring_error[256];

int32_t ring_fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_ring_error, sizeof(g_ring_error), fmt, ap);
  va_end(ap);
  return code;
}

int64_t chunk_slots(const mla_ring* r) { return (int64_t)r->sink_chunks + r->window_chunks + 1; }

// Chunk slot of chunk j.
int64_t slot_of(const mla_ring* r, int64_t j) {
  if (j < r->sink_chunks) return j;
  return r->sink_chunks + (j - r->sink_chunks) % ((int64_t)r->window_chunks + 1);
}

int32_t check_ring(const mla_ring* r) {
  if (r == nullptr) return ring_fail(MLA_ERR_INVALID_ARG, "ring is null");
  if (r->chunk_tokens < 1 || r->sink_chunks < 0 || r->window_chunks < 0 || r->committed < 0)
    return ring_fail(MLA_ERR_INVALID_ARG, "ring state is invalid");
  return MLA_OK;
}
}  // namespace

extern "C" {

int32_t mla_ring_init(mla_ring* r, int32_t chunk_tokens, int32_t sink_chunks, int32_t window_chunks) {
  if (r == nullptr) return ring_fail(MLA_ERR_INVALID_ARG, "ring is null");
  if (chunk_tokens < 1 || sink_chunks < 0 || window_chunks < 0)
    return ring_fail(MLA_ERR_INVALID_ARG, "chunk_tokens must be >= 1, sink_chunks and window_chunks >= 0");
  const int64_t cap = ((int64_t)sink_chunks + window_chunks + 1) * chunk_tokens;
  if (cap > INT32_MAX) return ring_fail(MLA_ERR_UNSUPPORTED, "ring capacity %lld exceeds int32", (long long)cap);
  r->chunk_tokens = chunk_tokens;
  r->sink_chunks = sink_chunks;
  r->window_chunks = window_chunks;
  r->capacity = (int32_t)cap;
  r->committed = 0;
  return MLA_OK;
}

int32_t mla_ring_current(const mla_ring* r, int32_t* write_offset, int32_t* n_k) {
  int32_t st = check_ring(r);
  if (st) return st;
  if (write_offset == nullptr || n_k == nullptr) return ring_fail(MLA_ERR_INVALID_ARG, "output pointer is null");
  const int64_t k = r->committed;
  const int64_t live = k + 1 < chunk_slots(r) ? k + 1 : chunk_slots(r);
  *write_offset = (int32_t)(slot_of(r, k) * r->chunk_tokens);
  *n_k = (int32_t)(live * r->chunk_tokens);
  return MLA_OK;
}

int32_t mla_ring_commit(mla_ring* r) {
  int32_t st = check_ring(r);
  if (st) return st;
  r->committed += 1;
  return MLA_OK;
}

int32_t mla_ring_slot_chunks(const mla_ring* r, int64_t* chunk_of_slot) {
  int32_t st = check_ring(r);
  if (st) return st;
  if (chunk_of_slot == nullptr) return ring_fail(MLA_ERR_INVALID_ARG, "chunk_of_slot is null");
  const int64_t S = chunk_slots(r), k = r->committed;
  for (int64_t s = 0; s < S; ++s) chunk_of_slot[s] = -1;
  // sinks, then the window chunks still cached, then the current chunk
  const int64_t first_window = k - r->window_chunks > r->sink_chunks ? k - r->window_chunks : r->sink_chunks;
  for (int64_t j = 0; j < r->sink_chunks && j <= k; ++j) chunk_of_slot[slot_of(r, j)] = j;
  for (int64_t j = first_window; j <= k; ++j) chunk_of_slot[slot_of(r, j)] = j;
  return MLA_OK;
}

int64_t mla_cache_bytes(const mla_dims* dims, int32_t dtype, int32_t capacity) {
  if (dims == nullptr || capacity < 0 || (dtype != MLA_BF16 && dtype != MLA_F32))
    return ring_fail(MLA_ERR_INVALID_ARG, "invalid arguments");
  return (int64_t)dims->batch * capacity * (dims->d_c + dims->d_r) * (dtype == MLA_F32 ? 4 : 2);
}

int64_t mla_dense_kv_bytes(const mla_dims* dims, int32_t dtype, int32_t capacity) {
  if (dims == nullptr || capacity < 0 || (dtype != MLA_BF16 && dtype != MLA_F32))
    return ring_fail(MLA_ERR_INVALID_ARG, "invalid arguments");
  return (int64_t)dims->batch * capacity * 2 * dims->n_heads * dims->head_dim * (dtype == MLA_F32 ? 4 : 2);
}

const char* mla_ring_last_error(void) { return g_ring_error; }

}  // extern "C"
