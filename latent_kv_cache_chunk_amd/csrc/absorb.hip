// Query absorption: the per-head key up-projection is folded into the query,
//   q~[b][h*n_q + i] = qscale * [ W_UK[h]^T q[b,i,h]  ||  RoPE3D(p_i) q_r[b,i,h] ],
// qscale = softmax_scale * log2(e), rounded once to the storage dtype.
// Scores are then taken directly against the cached latent rows [c || k_R]
// (multi-head latent attention, DeepSeek-V2, listed under "Builds on" on the
// VideoMLA mlsanity.com page; decoupled positional query per head with one
// head-shared rotated key: VideoMLA arXiv abstract).
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Rotation of every (query, rotary pair): cos and sin of the fp64 angle,
// rounded to fp32 once; shared by all heads and batch samples.
__global__ __launch_bounds__(256)
void rope_table_kernel(const int* __restrict__ q_pos, int n_q, int pairs, RopeSpec rope, f32x2* __restrict__ cs) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_q * pairs) return;
  const int i = idx / pairs, pr = idx - i * pairs;
  const double ang = rope_angle(pr, q_pos[3 * i], q_pos[3 * i + 1], q_pos[3 * i + 2], rope);
  cs[idx] = f32x2{(float)cos(ang), (float)sin(ang)};
}

// One workgroup = 4 wavefronts = 128 queries of one (batch, head).
// Content part on MFMA: C^T[c][i] = sum_d W_UK[h][d][c] q[i][d].  W_UK[h]
// (128 x d_c) is staged once in LDS, rows padded to an odd number of 16-byte
// slots, and its transpose is read as the A operand with ds_read_tr16_b64
// (two reads give a lane eight d of one column c).  Those eight d are
// {4h..4h+3, 8+4h..8+4h+3} of the 16-wide k-step for lane half h, so the B
// operand takes q in the same order (two 8-byte loads).  The rotated
// positional part comes from the (cos, sin) table.
template <int DC>
__global__ __launch_bounds__(256)
void absorb_bf16_kernel(const u16* __restrict__ q, const u16* __restrict__ q_r,
                        const f32x2* __restrict__ rope_cs, int n_q, int H,
                        const u16* __restrict__ w_uk, float qscale,
                        u16* __restrict__ qt, int rows_pad_b) {
  constexpr int DH = 128, DR = 32, W = DC + DR, CB = DC / 32;
  constexpr int NCH = DC / 8, ROWB = (NCH + 1) * 16;
  static_assert((NCH + 1) & 1, "odd slot stride");
  __shared__ __attribute__((aligned(16))) char wl[DH * ROWB];
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int i = blockIdx.y * 128 + wave * 32 + (lane & 31);
  const bool ok = i < n_q;

  const u16* wk = w_uk + (int64_t)h * DH * DC;
  for (int idx = threadIdx.x; idx < DH * NCH; idx += 256) {
    const int r = idx / NCH, ch = idx - r * NCH;
    *reinterpret_cast<uint4*>(wl + r * ROWB + ch * 16) = *reinterpret_cast<const uint4*>(wk + r * DC + ch * 8);
  }

  const int64_t qrow_off = (((int64_t)b * n_q + (ok ? i : 0)) * H + h);
  const u16* qrow = q + qrow_off * DH + half * 4;
  bf16x8 qf[DH / 16];
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks) {
    const uint2 lo = ok ? *reinterpret_cast<const uint2*>(qrow + ks * 16) : make_uint2(0, 0);
    const uint2 hi = ok ? *reinterpret_cast<const uint2*>(qrow + ks * 16 + 8) : make_uint2(0, 0);
    qf[ks] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  __syncthreads();

  const int g = lane >> 4, j = lane & 15;
  const char* abase = wl + ((g >> 1) * 4 + (j >> 2)) * ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;
  u16* orow = qt + ((int64_t)b * rows_pad_b + (int64_t)h * n_q + i) * W;
#pragma unroll 1
  for (int cb = 0; cb < CB; ++cb) {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const char* ab = abase + ks * 16 * ROWB + cb * 64;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)ab);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ab + 8 * ROWB));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = mfma_32x32x16(a, qf[ks], acc);
    }
    if (ok) {
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int c0 = cb * 32 + gg * 8 + half * 4;
        const uint32_t lo = bf16x2_bits(to_bf16x2(acc[4 * gg] * qscale, acc[4 * gg + 1] * qscale));
        const uint32_t hi = bf16x2_bits(to_bf16x2(acc[4 * gg + 2] * qscale, acc[4 * gg + 3] * qscale));
        *reinterpret_cast<uint2*>(orow + c0) = make_uint2(lo, hi);
      }
    }
  }

  // Positional part: lane half `half` rotates pairs 8*half .. 8*half+7.
  if (ok) {
    const u16* qr = q_r + qrow_off * DR + half * 16;
    const f32x2* cs = rope_cs + (int64_t)i * (DR / 2) + half * 8;
    uint32_t outw[8];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const float x0 = (float)__builtin_bit_cast(__bf16, qr[2 * pp]);
      const float x1 = (float)__builtin_bit_cast(__bf16, qr[2 * pp + 1]);
      const f32x2 r = cs[pp];
      const float y0 = fmaf(x0, r[0], -(x1 * r[1])), y1 = fmaf(x0, r[1], x1 * r[0]);
      outw[pp] = bf16x2_bits(to_bf16x2(y0 * qscale, y1 * qscale));
    }
    uint4* o = reinterpret_cast<uint4*>(orow + DC + half * 16);
    o[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    o[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
  }

  // Padding rows after the last real row of each sample are zero so that the
  // attention kernel reads only finite values.
  if (h == 0 && blockIdx.y == 0) {
    const int rows_b = H * n_q;
    u16* pad = qt + ((int64_t)b * rows_pad_b + rows_b) * W;
    const int64_t n = (int64_t)(rows_pad_b - rows_b) * W / 8;
    for (int64_t k = threadIdx.x; k < n; k += blockDim.x)
      reinterpret_cast<uint4*>(pad)[k] = make_uint4(0, 0, 0, 0);
  }
}

// fp32 variant: thread per (row, output column); content columns are plain
// dot products over d, positional columns are handled as pairs.
__global__ __launch_bounds__(256)
void absorb_f32_kernel(const float* __restrict__ q, const float* __restrict__ q_r,
                       const int* __restrict__ q_pos, int n_q, int H, int DC,
                       const float* __restrict__ w_uk, float qscale,
                       float* __restrict__ qt, int rows_pad_b, int B, RopeSpec rope) {
  constexpr int DH = 128, DR = 32;
  const int W = DC + DR;
  const int cols = DC + DR / 2;                 // DC content columns + 16 pairs
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)B * rows_pad_b;
  if (idx >= rows * cols) return;
  const int64_t row = idx / cols;
  const int col = (int)(idx - row * cols);
  const int b = (int)(row / rows_pad_b);
  const int r = (int)(row - (int64_t)b * rows_pad_b);
  float* orow = qt + row * W;
  if (r >= H * n_q) {                            // padding row
    if (col < DC) orow[col] = 0.f;
    else { orow[DC + 2 * (col - DC)] = 0.f; orow[DC + 2 * (col - DC) + 1] = 0.f; }
    return;
  }
  const int h = r / n_q, i = r - h * n_q;
  const int64_t qoff = ((int64_t)b * n_q + i) * H + h;
  if (col < DC) {
    const float* qv = q + qoff * DH;
    const float* wk = w_uk + (int64_t)h * DH * DC + col;
    float acc = 0.f;
    for (int d = 0; d < DH; ++d) acc = fmaf(qv[d], wk[(int64_t)d * DC], acc);
    orow[col] = acc * qscale;
  } else {
    const int pair = col - DC;
    const float* qr = q_r + qoff * DR;
    const float x0 = qr[2 * pair], x1 = qr[2 * pair + 1];
    const double ang = rope_angle(pair, q_pos[3 * i], q_pos[3 * i + 1], q_pos[3 * i + 2], rope);
    const float cs = (float)cos(ang), sn = (float)sin(ang);
    orow[DC + 2 * pair] = fmaf(x0, cs, -(x1 * sn)) * qscale;
    orow[DC + 2 * pair + 1] = fmaf(x0, sn, x1 * cs) * qscale;
  }
}

hipError_t launch_absorb_bf16(const Plan& p, const AbsorbArgs& a, hipStream_t s) {
  const int pairs = (p.width - p.d_c) / 2;
  f32x2* cs = (f32x2*)a.rope_cs;
  rope_table_kernel<<<dim3((unsigned)((p.n_q * pairs + 255) / 256)), dim3(256), 0, s>>>(a.q_pos, p.n_q, pairs, a.rope,
                                                                                         cs);
  const dim3 grid(p.B * p.H, (p.n_q + 127) / 128), block(256);
  const u16* q = (const u16*)a.q;
  const u16* qr = (const u16*)a.q_r;
  const u16* wk = (const u16*)a.w_uk;
  u16* qt = (u16*)a.qt;
  switch (p.d_c) {
    case 64: absorb_bf16_kernel<64><<<grid, block, 0, s>>>(q, qr, cs, p.n_q, p.H, wk, a.qscale, qt, p.rows_pad_b); break;
    case 128: absorb_bf16_kernel<128><<<grid, block, 0, s>>>(q, qr, cs, p.n_q, p.H, wk, a.qscale, qt, p.rows_pad_b); break;
    case 192: absorb_bf16_kernel<192><<<grid, block, 0, s>>>(q, qr, cs, p.n_q, p.H, wk, a.qscale, qt, p.rows_pad_b); break;
    case 256: absorb_bf16_kernel<256><<<grid, block, 0, s>>>(q, qr, cs, p.n_q, p.H, wk, a.qscale, qt, p.rows_pad_b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_absorb_f32(const Plan& p, const AbsorbArgs& a, hipStream_t s) {
  const int cols = p.d_c + 16;
  const int64_t work = (int64_t)p.B * p.rows_pad_b * cols;
  const dim3 grid((unsigned)((work + 255) / 256)), block(256);
  absorb_f32_kernel<<<grid, block, 0, s>>>((const float*)a.q, (const float*)a.q_r, a.q_pos, p.n_q,
                                           p.H, p.d_c, (const float*)a.w_uk, a.qscale,
                                           (float*)a.qt, p.rows_pad_b, p.B, a.rope);
  return hipGetLastError();
}

}  // namespace mla
