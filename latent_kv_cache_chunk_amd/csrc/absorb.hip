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

// 2*pi as an fp64 pair (high part + remainder) and 1/(2*pi), for reducing
// RoPE angles to [-pi, pi] before the fp32 sine and cosine.
constexpr double kTwoPiHi = 6.283185307179586232;
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189533577;

// One workgroup = 4 wavefronts = 128 queries of one (batch, head).
// Content part on MFMA: C^T[c][i] = sum_d W_UK[h][d][c] q[i][d].  W_UK[h]
// (128 x d_c) is staged once in LDS, rows padded to an odd number of 16-byte
// slots, and its transpose is read as the A operand with ds_read_tr16_b64
// (two reads give a lane eight d of one column c).  Those reads hand lane
// half h the LDS rows {4h..4h+3, 8+4h..8+4h+3} of each 16-row k-step, so
// W_UK row d is staged in LDS row d with bits 2 and 3 swapped: lane half h
// then holds d = 8h .. 8h+7 in order, and q is loaded as one 16-byte piece
// per k-step.  The rotated positional part comes from the (cos, sin) table.
// Finished rows go through LDS (over the W_UK stage, after a barrier): a
// wavefront's 32 rows of q~ are contiguous in memory and leave as whole
// 16-byte pieces of consecutive addresses.
//
// The positional part rotates q_r by RoPE3D(p_i): the angle p_a * theta^(-2k/d_a)
// of each pair is formed in fp64 (the 16 inverse frequencies once per
// workgroup, in LDS), reduced exactly to [-pi, pi] with a two-part 2*pi, and
// its sine and cosine are taken in fp32.  Their error (about one fp32 ulp) is
// far below the bf16 rounding of q~ that follows.
//
// Workgroup id -> (sample b, head h, query block y): a 128-byte line of q_r
// holds two heads' 32 values, so the heads 2k and 2k+1 of one query block get
// ids 8 apart -- the same XCD (workgroups are dealt to the eight XCDs round
// robin) and neighbours in its dispatch order -- and the line is fetched into
// one L2 once.  Units u = (b * ceil(H/2) + k) * NY + y; id = 16*(u/8) +
// 8*(h%2) + u%8.
template <int DC>
__global__ __launch_bounds__(256)
void absorb_bf16_kernel(const u16* __restrict__ q, const u16* __restrict__ q_r,
                        const int* __restrict__ q_pos, RopeSpec rope, int n_q, int H, int B,
                        const u16* __restrict__ w_uk, float qscale,
                        u16* __restrict__ qt, int rows_pad_b) {
  constexpr int DH = 128, DR = 32, W = DC + DR, CB = DC / 32;
  constexpr int NCH = DC / 8, ROWB = (NCH + 1) * 16;
  static_assert((NCH + 1) & 1, "odd slot stride");
  constexpr int OROW = W * 2 + 16;                       // staged output row (odd number of 16-byte slots)
  static_assert(((W * 2 + 16) / 16) & 1, "odd slot stride");
  constexpr int WBYTES = DH * ROWB, OBYTES = 4 * 32 * OROW;
  __shared__ __attribute__((aligned(16))) char wl[WBYTES > OBYTES ? WBYTES : OBYTES];
  __shared__ double rope_ifreq[DR / 2];
  __shared__ int rope_axis[DR / 2];
  const int ny = (n_q + 127) / 128, hp = (H + 1) / 2;
  const int u = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
  const int y = u % ny, bk = u / ny, b = bk / hp;
  const int h = 2 * (bk - b * hp) + ((blockIdx.x >> 3) & 1);
  if (b >= B || h >= H) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int i0 = y * 128 + wave * 32;                    // first query of this wavefront
  const int i = i0 + (lane & 31);
  const bool ok = i < n_q;

  if (threadIdx.x < DR / 2) {
    int axis;
    rope_ifreq[threadIdx.x] = rope_inv_freq(threadIdx.x, rope, axis);
    rope_axis[threadIdx.x] = axis;
  }
  // A thread's pieces of W_UK[h] and its q row are all loaded before the first
  // LDS store, so the staging costs one round trip, not one per piece.
  constexpr int PER = DH * NCH / 256;                    // 16-byte pieces per thread
  static_assert(DH * NCH % 256 == 0, "whole pieces per thread");
  const u16* wk = w_uk + (int64_t)h * DH * DC;
  uint4 wv[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = threadIdx.x + 256 * k, r = idx / NCH, ch = idx - r * NCH;
    wv[k] = *reinterpret_cast<const uint4*>(wk + r * DC + ch * 8);
  }
  const int ic = ok ? i : 0;
  const int64_t qrow_off = (((int64_t)b * n_q + ic) * H + h);
  const u16* qrow = q + qrow_off * DH + half * 8;
  bf16x8 qf[DH / 16];
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks)
    qf[ks] = ok ? *reinterpret_cast<const bf16x8*>(qrow + ks * 16) : bf16x8{};
  // The positional inputs (this lane half's 16 q_r values and the query's
  // position) load with the rest, so the rotation after the product does not
  // wait on another round trip.
  const u16* qr = q_r + qrow_off * DR + half * 16;
  uint4 r0 = *reinterpret_cast<const uint4*>(qr), r1 = *reinterpret_cast<const uint4*>(qr + 8);
  int pt = q_pos[3 * ic], ph = q_pos[3 * ic + 1], pw = q_pos[3 * ic + 2];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = threadIdx.x + 256 * k, r = idx / NCH, ch = idx - r * NCH;
    const int rs = (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
    *reinterpret_cast<uint4*>(wl + rs * ROWB + ch * 16) = wv[k];
  }
  // pin that order (the scheduler otherwise pairs each load with its store)
  __builtin_amdgcn_sched_group_barrier(0x020, PER + DH / 16 + 5, 0);
  __builtin_amdgcn_sched_group_barrier(0x200, PER, 0);
  // Keeps the positional loads here (the compiler would otherwise sink them to
  // their use after the product); every load of the thread has landed by the
  // barrier below anyway.
  asm volatile("" : "+v"(r0.x), "+v"(r0.y), "+v"(r0.z), "+v"(r0.w), "+v"(r1.x), "+v"(r1.y), "+v"(r1.z),
               "+v"(r1.w), "+v"(pt), "+v"(ph), "+v"(pw));
  __syncthreads();

  const int g = lane >> 4, j = lane & 15;
  const char* abase = wl + ((g >> 1) * 4 + (j >> 2)) * ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    acc[cb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const char* ab = abase + ks * 16 * ROWB + cb * 64;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)ab);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ab + 8 * ROWB));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[cb] = mfma_32x32x16(a, qf[ks], acc[cb]);
    }
  }
  __syncthreads();   // every wavefront is done with the W_UK stage

  // this wavefront's 32 output rows, staged in LDS
  char* orow = wl + wave * 32 * OROW + (lane & 31) * OROW;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int c0 = cb * 32 + gg * 8 + half * 4;
      const uint32_t lo = bf16x2_bits(to_bf16x2(acc[cb][4 * gg] * qscale, acc[cb][4 * gg + 1] * qscale));
      const uint32_t hi = bf16x2_bits(to_bf16x2(acc[cb][4 * gg + 2] * qscale, acc[cb][4 * gg + 3] * qscale));
      *reinterpret_cast<uint2*>(orow + c0 * 2) = make_uint2(lo, hi);
    }
  // Positional part: lane half `half` rotates pairs 8*half .. 8*half+7.
  if (ok) {
    const uint32_t in[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    uint32_t outw[8];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      const float x0 = __builtin_bit_cast(float, in[pp] << 16);
      const float x1 = __builtin_bit_cast(float, in[pp] & 0xFFFF0000u);
      const int pr = half * 8 + pp;
      const int ax = rope_axis[pr];
      const double ang = (double)(ax == 0 ? pt : ax == 1 ? ph : pw) * rope_ifreq[pr];
      const double k = rint(ang * kInvTwoPi);
      const float red = (float)fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
      float sn, cs;
      sincosf(red, &sn, &cs);
      const float y0 = fmaf(x0, cs, -(x1 * sn)), y1 = fmaf(x0, sn, x1 * cs);
      outw[pp] = bf16x2_bits(to_bf16x2(y0 * qscale, y1 * qscale));
    }
    uint4* o = reinterpret_cast<uint4*>(orow + (DC + half * 16) * 2);
    o[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    o[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
  }
  // the wavefront's LDS accesses run in order; these keep the compiler from
  // moving the copy-out reads above other lanes' writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // copy-out: rows h*n_q + i0 .. of this sample are consecutive in q~
  const int nrows = min(32, n_q - i0);
  if (nrows > 0) {
    constexpr int PIECES = W * 2 / 16;                   // 16-byte pieces per row
    char* dst = reinterpret_cast<char*>(qt + ((int64_t)b * rows_pad_b + (int64_t)h * n_q + i0) * W);
    const char* src = wl + wave * 32 * OROW;
    for (int pc = lane; pc < nrows * PIECES; pc += 64) {
      const int row = pc / PIECES, col = pc - row * PIECES;
      *reinterpret_cast<uint4*>(dst + (int64_t)pc * 16) = *reinterpret_cast<const uint4*>(src + row * OROW + col * 16);
    }
  }

  // Padding rows after the last real row of each sample are zero so that the
  // attention kernel reads only finite values.
  if (h == 0 && y == 0) {
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
  const int64_t units = (int64_t)p.B * ((p.H + 1) / 2) * ((p.n_q + 127) / 128);
  const dim3 grid((unsigned)((units + 7) / 8 * 16)), block(256);   // see the id mapping in the kernel
  const u16* q = (const u16*)a.q;
  const u16* qr = (const u16*)a.q_r;
  const u16* wk = (const u16*)a.w_uk;
  u16* qt = (u16*)a.qt;
  switch (p.d_c) {
    case 64: absorb_bf16_kernel<64><<<grid, block, 0, s>>>(q, qr, a.q_pos, a.rope, p.n_q, p.H, p.B, wk, a.qscale, qt, p.rows_pad_b); break;
    case 128: absorb_bf16_kernel<128><<<grid, block, 0, s>>>(q, qr, a.q_pos, a.rope, p.n_q, p.H, p.B, wk, a.qscale, qt, p.rows_pad_b); break;
    case 192: absorb_bf16_kernel<192><<<grid, block, 0, s>>>(q, qr, a.q_pos, a.rope, p.n_q, p.H, p.B, wk, a.qscale, qt, p.rows_pad_b); break;
    case 256: absorb_bf16_kernel<256><<<grid, block, 0, s>>>(q, qr, a.q_pos, a.rope, p.n_q, p.H, p.B, wk, a.qscale, qt, p.rows_pad_b); break;
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
