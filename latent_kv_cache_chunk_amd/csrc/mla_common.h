// Shared device helpers and the workspace plan of the latent-attention path.
// gfx950 (CDNA4) only: 64-wide wavefronts, bf16 MFMA 32x32x16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace mla {

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Rows of (batch, head, query) handled by one attention workgroup.
constexpr int kRowsPerBlock = 256;
// Keys per latent tile staged in LDS.  d_c <= 192 (attend.hip): three key
// buffers and two P buffers (16 KB per 32 keys) fit the 160 KB of LDS with
// 64-key tiles.  d_c = 256 (attend_wide.hip): two 128-key buffers.
__host__ __device__ constexpr int key_tile(int d_c) { return d_c <= 192 ? 64 : 128; }
// Compute units the work partition is sized for (MI355X).
constexpr int kPartitionCUs = 256;
// Start-up cost of a row-block segment, in key tiles of work, for the
// partition of chunk-causal calls: loading the rows' queries, filling and
// draining the tile pipeline, writing the partial state (and merging it
// afterwards).  Counting it evens out workgroups that cover many short row
// blocks against those that cover a few long ones.  At 7 chunks of 4680
// queries a probe build timed each segment's sweep at 5.9 us + 2.53 us per
// tile, with 3.0 us before it and 5.6 us after it: about 14.5 us, six tiles,
// of fixed cost.  Kernel times over the values 4..24 are flat from 12 to 24
// (the merge's extra states and the row blocks' L2 drift also grow with the
// segment count), and 16 sits in the middle.
constexpr int kSegmentUnits = 16;
// Workgroups per row block, at most, on average: G <= kMaxSplitsPerBlock *
// nrb.  Short chunks (few row blocks) would otherwise spread each row block
// over up to a hundred workgroups and leave the merge that many partial
// states per row.  (Equal row blocks then meet at most 17 workgroups each;
// a long row block of a chunk-causal call can meet a few more.)
constexpr int kMaxSplitsPerBlock = 16;
// log2(e): softmax runs in base 2 with this folded into the query scale.
constexpr double kLog2e = 1.4426950408889634074;

// ---------------------------------------------------------------------------
// Chunk-causal visibility.  Query i of a call is token q_start + i of the key
// sequence; with chunk length C it sees keys [0, kv(i)) where
//   kv(i) = min(n_k, (floor((q_start + i) / C) + 1) * C)
// (every earlier chunk and its own chunk, bidirectionally).  chunk_len == 0:
// every query sees all n_k keys.  Rows are r = h * n_q + i per sample; rows
// past H * n_q are padding and see one key (their output is never read).
// ---------------------------------------------------------------------------
struct Visibility {
  int n_q, rows_b, q_start, chunk_len;

  __host__ __device__ int kv_of_row(int r, int n_k) const {
    if (chunk_len == 0) return n_k;
    if (r >= rows_b) return 1;
    const int i = r % n_q;
    return min(n_k, ((q_start + i) / chunk_len + 1) * chunk_len);
  }
  // Largest kv over rows [r0, r0 + nrows) (kv grows with i inside a head, so
  // the last row decides unless the range crosses into a new head).
  __host__ __device__ int kv_max_of_rows(int r0, int nrows, int n_k) const {
    if (chunk_len == 0) return n_k;
    const int r1 = min(r0 + nrows, rows_b) - 1;
    if (r1 < r0) return 1;
    return (r0 / n_q != r1 / n_q) ? kv_of_row((r0 / n_q) * n_q + n_q - 1, n_k) : kv_of_row(r1, n_k);
  }
  __host__ __device__ int kv_max_of_block(int r0, int n_k) const { return kv_max_of_rows(r0, kRowsPerBlock, n_k); }
};

// ---------------------------------------------------------------------------
// Work partition of the fused attention kernel.
//
// Units are (row-block, key-tile) pairs.  Every key tile of a row block is a
// unit (T per row block) unless the call is chunk-causal and its row blocks
// see different numbers of key tiles: then a row block has kSegmentUnits
// start-up units (no tile) followed by the tiles some of its rows can see,
// and units[rb] (an exclusive prefix sum, in the workspace) gives the first
// unit of row block rb; unit first + kSegmentUnits + t is its tile t
// (seg_tiles below).  G workgroups each take the contiguous unit
// range [floor(w*U/G), floor((w+1)*U/G)) and leave one partial softmax state
// per row block whose tiles they touch, in slot w + rb: a workgroup's row
// blocks are consecutive, so these slots are distinct, and fewer than
// G + nrb.  The merge step finds the owners of a row block's first key-tile
// unit and of its last unit arithmetically; every workgroup between them
// holds some of the row block's tiles (ranges are never empty, as G <= U).
//
// A slot holds, for its 256 rows, (m, l) pairs and the unnormalised fp32 L
// rows.  The bf16 kernels store L channel-quad-major inside each 32-row
// group: float index part_L_index(slot, row, c) below, so that one 16-byte
// store or load of a wavefront (32 rows, one channel quad per lane half)
// covers two contiguous 512-byte runs.  The fp32 kernels keep plain rows.
// ---------------------------------------------------------------------------
struct Plan {
  int32_t B, H, n_q, n_k, d_c, width;   // width = d_c + d_r
  int32_t rows_b;       // H * n_q real rows per sample (row = h*n_q + i)
  int32_t rb_per_b;     // row-blocks per sample
  int32_t rows_pad_b;   // rb_per_b * kRowsPerBlock
  int32_t nrb;          // B * rb_per_b
  int32_t T;            // key tiles
  int64_t U;            // units
  int32_t G;            // attention workgroups
  bool causal;          // per-row-block units (chunk-causal call)
  int32_t elem;         // bytes per element of q~ (2 bf16, 4 f32)
  // byte offsets inside the workspace
  int64_t off_qt, off_L, off_ml, off_units, off_hdr, total;
};

// The partition the attention kernel used, left in the workspace for the merge.
struct PartitionHeader {
  int64_t U;
  int32_t G;
  int32_t per_block_units;   // 1: units[] holds each row block's first unit; 0: row block rb starts at rb * T
};

__host__ __device__ inline int64_t unit_begin(int64_t w, int64_t U, int64_t G) {
  return (w * U) / G;
}
// Workgroup that owns unit u: the largest w with floor(w*U/G) <= u.
__host__ __device__ inline int64_t unit_owner(int64_t u, int64_t U, int64_t G) {
  return ((u + 1) * G - 1) / U;
}
// First unit of row block rb (units == nullptr: T units per row block).
__host__ __device__ inline int64_t rb_first_unit(const int64_t* units, int64_t T, int64_t rb) {
  return units ? units[rb] : rb * T;
}
// Row block holding unit u: the largest rb with rb_first_unit(rb) <= u.
__host__ __device__ inline int64_t rb_of_unit(const int64_t* units, int64_t T, int64_t nrb, int64_t u) {
  if (units == nullptr) return u / T;
  int64_t lo = 0, hi = nrb - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (units[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}
// First unit of row block rb that holds a key tile (the start-up units of a
// chunk-causal row block hold none).  A workgroup whose part of a row block
// is start-up units only leaves no partial state for it, so the merge starts
// at the owner of this unit.
__host__ __device__ inline int64_t rb_first_tile_unit(const int64_t* units, int64_t T, int64_t rb) {
  return rb_first_unit(units, T, rb) + (units ? kSegmentUnits : 0);
}
// Tiles [t0, t1) of the units [begin, end) of a row block whose first unit is
// `first` (start-up units of chunk-causal row blocks hold no tile).
__host__ __device__ inline void seg_tiles(const int64_t* units, int64_t first, int64_t begin, int64_t end, int& t0,
                                          int& t1) {
  const int64_t skip = units ? kSegmentUnits : 0;
  t0 = (int)(begin - first - skip > 0 ? begin - first - skip : 0);
  t1 = (int)(end - first - skip > 0 ? end - first - skip : 0);
}
// Slot of workgroup w's partial state for row block rb.
__host__ __device__ inline int64_t seg_slot(int64_t w, int64_t rb) { return w + rb; }
// Float index of channel c of row `row` (0..255) of a slot's L (bf16 kernels):
// [row / 32][c / 4][row % 32][c % 4] inside the slot.
__host__ __device__ inline int64_t part_L_index(int64_t slot, int row, int c, int d_c) {
  return (slot * kRowsPerBlock + (row & ~31)) * d_c + (c >> 2) * 128 + (row & 31) * 4 + (c & 3);
}

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Build the plan.  bf16: stream-K style partition over kPartitionCUs when the
// plain one-workgroup-per-row-block launch would leave more than 10% of the
// compute units idle in its last round; chunk-causal calls whose row blocks
// see different numbers of key tiles always spread their units over
// kPartitionCUs workgroups; either way G is at most kMaxSplitsPerBlock per
// row block.  f32: one workgroup per row-block.  The workspace size does not
// depend on `vis`.
inline Plan make_plan(int B, int H, int n_q, int n_k, int d_c, int d_r, bool f32,
                      const Visibility* vis = nullptr) {
  Plan p{};
  p.B = B; p.H = H; p.n_q = n_q; p.n_k = n_k; p.d_c = d_c; p.width = d_c + d_r;
  p.rows_b = H * n_q;
  p.rb_per_b = (p.rows_b + kRowsPerBlock - 1) / kRowsPerBlock;
  p.rows_pad_b = p.rb_per_b * kRowsPerBlock;
  p.nrb = B * p.rb_per_b;
  const int bn = key_tile(d_c);
  p.T = (n_k + bn - 1) / bn;
  p.U = (int64_t)p.nrb * p.T;
  p.elem = f32 ? 4 : 2;
  int64_t G = p.nrb;
  if (!f32) {
    int64_t rounds = (p.nrb + kPartitionCUs - 1) / kPartitionCUs;
    double eff = (double)p.nrb / (double)(rounds * kPartitionCUs);
    if (eff < 0.9) G = rounds * kPartitionCUs;
    if (G > p.U) G = p.U;
    if (G > (int64_t)p.nrb * kMaxSplitsPerBlock) G = (int64_t)p.nrb * kMaxSplitsPerBlock;
  }
  // Slots for the workgroups' partial states: enough for this G and for the G
  // of any chunk-causal call of the same sizes (at most min(kPartitionCUs,
  // nrb * kMaxSplitsPerBlock)), so the workspace size does not depend on `vis`.
  const int64_t causal_g = std::min<int64_t>(kPartitionCUs, (int64_t)p.nrb * kMaxSplitsPerBlock);
  const int64_t g_slots = G > causal_g ? G : causal_g;
  // A chunk-causal call in which every row block sees every key tile keeps
  // the plain partition (its rows still mask their own keys), so that it
  // splits the keys exactly as the unmasked call does.
  bool uneven = false;
  if (!f32 && vis != nullptr && vis->chunk_len != 0)
    for (int rbl = 0; rbl < p.rb_per_b && !uneven; ++rbl)
      uneven = (vis->kv_max_of_block(rbl * kRowsPerBlock, n_k) + bn - 1) / bn != p.T;
  if (uneven) {
    int64_t per_b = 0;
    for (int rbl = 0; rbl < p.rb_per_b; ++rbl)
      per_b += (vis->kv_max_of_block(rbl * kRowsPerBlock, n_k) + bn - 1) / bn + kSegmentUnits;
    p.U = (int64_t)B * per_b;
    G = p.U < kPartitionCUs ? p.U : kPartitionCUs;
    if (G > (int64_t)p.nrb * kMaxSplitsPerBlock) G = (int64_t)p.nrb * kMaxSplitsPerBlock;
    p.causal = true;
  }
  p.G = (int32_t)G;
  const int64_t slots = f32 ? (int64_t)p.nrb : g_slots + p.nrb;
  p.off_qt = 0;
  int64_t qt_bytes = (int64_t)B * p.rows_pad_b * p.width * p.elem;
  p.off_L = align_up(qt_bytes, 256);
  int64_t L_bytes = slots * kRowsPerBlock * (int64_t)d_c * 4;
  p.off_ml = align_up(p.off_L + L_bytes, 256);
  int64_t ml_bytes = slots * kRowsPerBlock * 2 * 4;
  p.off_units = align_up(p.off_ml + ml_bytes, 256);
  p.off_hdr = align_up(p.off_units + (int64_t)(p.nrb + 1) * 8, 256);
  p.total = align_up(p.off_hdr + (int64_t)sizeof(PartitionHeader), 256);
  return p;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ inline f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32).
__device__ inline bf16x2 to_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

__device__ inline uint32_t bf16x2_bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// 3D-RoPE axis widths (contiguous blocks [t | h | w] of the d_r vector) and base.
struct RopeSpec {
  int t, h, w;
  double theta;
};

// Axis (0: t, 1: h, 2: w) and inverse frequency of 3D-RoPE pair `pair` (0 ..
// d_r/2-1), in fp64: pair i of an axis of width d_a turns by
// p_a * theta^(-2i/d_a).
__device__ inline double rope_inv_freq(int pair, const RopeSpec& r, int& axis) {
  const int e = 2 * pair;
  int width, i;
  if (e < r.t) { width = r.t; axis = 0; i = pair; }
  else if (e < r.t + r.h) { width = r.h; axis = 1; i = pair - r.t / 2; }
  else { width = r.w; axis = 2; i = pair - (r.t + r.h) / 2; }
  return pow(r.theta, -2.0 * (double)i / (double)width);
}

// Rotation angle of 3D-RoPE pair `pair` at position (t,h,w), in fp64.
__device__ inline double rope_angle(int pair, int pt, int ph, int pw, const RopeSpec& r) {
  int axis;
  const double inv_freq = rope_inv_freq(pair, r, axis);
  return (double)(axis == 0 ? pt : axis == 1 ? ph : pw) * inv_freq;
}

}  // namespace mla
