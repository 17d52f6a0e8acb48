// Shared device helpers and the workspace plan of the latent-attention path.
// gfx950 (CDNA4) only: 64-wide wavefronts, bf16 MFMA 32x32x16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// log2(e): softmax runs in base 2 with this folded into the query scale.
constexpr double kLog2e = 1.4426950408889634074;

// ---------------------------------------------------------------------------
// Work partition of the fused attention kernel.
//
// The (row-block, key-tile) space has U = nrb * T units.  G workgroups each
// take the contiguous unit range [floor(w*U/G), floor((w+1)*U/G)).  With
// G >= nrb a range is at most T units long, so it touches at most two
// row-blocks; the first row-block segment of workgroup w is stored in slot
// 2w and a second one in slot 2w+1.  A row-block whose units all belong to
// one workgroup still goes through a slot (one segment).  The combine step
// finds the owners of a row-block's first and last unit arithmetically.
// ---------------------------------------------------------------------------
struct Plan {
  int32_t B, H, n_q, n_k, d_c, width;   // width = d_c + d_r
  int32_t rows_b;       // H * n_q real rows per sample (row = h*n_q + i)
  int32_t rb_per_b;     // row-blocks per sample
  int32_t rows_pad_b;   // rb_per_b * kRowsPerBlock
  int32_t nrb;          // B * rb_per_b
  int32_t T;            // key tiles
  int64_t U;            // nrb * T
  int32_t G;            // attention workgroups
  int32_t elem;         // bytes per element of q~ (2 bf16, 4 f32)
  // byte offsets inside the workspace
  int64_t off_qt, off_L, off_ml, total;
};

__host__ __device__ inline int64_t unit_begin(int64_t w, int64_t U, int64_t G) {
  return (w * U) / G;
}
// Workgroup that owns unit u: the largest w with floor(w*U/G) <= u.
__host__ __device__ inline int64_t unit_owner(int64_t u, int64_t U, int64_t G) {
  return ((u + 1) * G - 1) / U;
}

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Build the plan.  bf16: stream-K style partition over kPartitionCUs when the
// plain one-workgroup-per-row-block launch would leave more than 10% of the
// compute units idle in its last round.  f32: one workgroup per row-block.
inline Plan make_plan(int B, int H, int n_q, int n_k, int d_c, int d_r, bool f32) {
  Plan p{};
  p.B = B; p.H = H; p.n_q = n_q; p.n_k = n_k; p.d_c = d_c; p.width = d_c + d_r;
  p.rows_b = H * n_q;
  p.rb_per_b = (p.rows_b + kRowsPerBlock - 1) / kRowsPerBlock;
  p.rows_pad_b = p.rb_per_b * kRowsPerBlock;
  p.nrb = B * p.rb_per_b;
  p.T = (n_k + key_tile(d_c) - 1) / key_tile(d_c);
  p.U = (int64_t)p.nrb * p.T;
  p.elem = f32 ? 4 : 2;
  int64_t G = p.nrb;
  if (!f32) {
    int64_t rounds = (p.nrb + kPartitionCUs - 1) / kPartitionCUs;
    double eff = (double)p.nrb / (double)(rounds * kPartitionCUs);
    if (eff < 0.9) G = rounds * kPartitionCUs;
    if (G > p.U) G = p.U;
  }
  p.G = (int32_t)G;
  const int64_t slots = f32 ? (int64_t)p.nrb : 2 * G;
  p.off_qt = 0;
  int64_t qt_bytes = (int64_t)B * p.rows_pad_b * p.width * p.elem;
  p.off_L = align_up(qt_bytes, 256);
  int64_t L_bytes = slots * kRowsPerBlock * (int64_t)d_c * 4;
  p.off_ml = align_up(p.off_L + L_bytes, 256);
  int64_t ml_bytes = slots * kRowsPerBlock * 2 * 4;
  p.total = align_up(p.off_ml + ml_bytes, 256);
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

// Rotation angle of 3D-RoPE pair `pair` (0 .. d_r/2-1) at position (t,h,w),
// evaluated in fp64: pair i of an axis of width d_a turns by p_a*theta^(-2i/d_a).
__device__ inline double rope_angle(int pair, int pt, int ph, int pw, const RopeSpec& r) {
  const int e = 2 * pair;
  int width, pos, i;
  if (e < r.t) { width = r.t; pos = pt; i = pair; }
  else if (e < r.t + r.h) { width = r.h; pos = ph; i = pair - r.t / 2; }
  else { width = r.w; pos = pw; i = pair - (r.t + r.h) / 2; }
  const double inv_freq = pow(r.theta, -2.0 * (double)i / (double)width);
  return (double)pos * inv_freq;
}

}  // namespace mla
