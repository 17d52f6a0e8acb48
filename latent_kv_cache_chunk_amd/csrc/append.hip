// Cache append: latent down-projection plus the rotated head-shared
// positional key, written as one [c || k_R] row per new token.
//
// VideoMLA (arXiv abstract, mlsanity.com paper page; atlas.scime.ai summary,
// "Approach"): each cached token keeps one content latent shared by all heads
// and one head-shared decoupled 3D-RoPE key.  The key is rotated here, once,
// so the cache already holds RoPE(p) k_R and attention never re-rotates keys.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One wavefront computes 32 tokens x all (d_c + d_r) outputs with bf16 MFMA
// 32x32x16, fp32 accumulation.  The product is formed transposed,
// C^T[n][token] = sum_k W[n][k] x[token][k], so each lane ends up holding
// four consecutive outputs of one token: RoPE pairs are lane-local and the
// bf16 store is 8 bytes.  Weight rows (n) are the A operand and are read
// straight from global memory (they stay in L2, the whole [W_DKV; W_KR] is
// 688 KB at D = 1536, d_c = 192); hidden states are the B operand.
template <int NB>
__global__ __launch_bounds__(64)
void append_bf16_kernel(const u16* __restrict__ x, int D, int ntok, int n_new,
                        const u16* __restrict__ w_dkv, const u16* __restrict__ w_kr, int d_c,
                        const int* __restrict__ pos, u16* __restrict__ cache, int cap, int off,
                        RopeSpec rope) {
  constexpr int W = NB * 32;
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int my_tok = blockIdx.x * 32 + (lane & 31);
  const bool tok_ok = my_tok < ntok;
  const u16* xrow = x + (int64_t)(tok_ok ? my_tok : 0) * D + half * 8;

  const u16* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 32 + (lane & 31);
    wrow[nb] = (n < d_c ? w_dkv + (int64_t)n * D : w_kr + (int64_t)(n - d_c) * D) + half * 8;
  }

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int k = 0; k < D; k += 16) {
    const bf16x8 bx = tok_ok ? *reinterpret_cast<const bf16x8*>(xrow + k)
                             : __builtin_bit_cast(bf16x8, zero);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 aw = *reinterpret_cast<const bf16x8*>(wrow[nb] + k);
      acc[nb] = mfma_32x32x16(aw, bx, acc[nb]);
    }
  }
  if (!tok_ok) return;

  const int b = my_tok / n_new, i = my_tok - b * n_new;
  u16* dst = cache + ((int64_t)b * cap + off + i) * W;
  const int pt = pos[3 * i + 0], ph = pos[3 * i + 1], pw = pos[3 * i + 2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n0 = nb * 32 + g * 8 + half * 4;       // 4 consecutive outputs
      float v0 = acc[nb][4 * g + 0], v1 = acc[nb][4 * g + 1];
      float v2 = acc[nb][4 * g + 2], v3 = acc[nb][4 * g + 3];
      if (n0 >= d_c) {                                  // positional key: rotate pairs
        const int pair = (n0 - d_c) >> 1;
        const double a0 = rope_angle(pair, pt, ph, pw, rope);
        const double a1 = rope_angle(pair + 1, pt, ph, pw, rope);
        const float c0 = (float)cos(a0), s0 = (float)sin(a0);
        const float c1 = (float)cos(a1), s1 = (float)sin(a1);
        const float r0 = fmaf(v0, c0, -(v1 * s0)), r1 = fmaf(v0, s0, v1 * c0);
        const float r2 = fmaf(v2, c1, -(v3 * s1)), r3 = fmaf(v2, s1, v3 * c1);
        v0 = r0; v1 = r1; v2 = r2; v3 = r3;
      }
      const uint32_t lo = bf16x2_bits(to_bf16x2(v0, v1));
      const uint32_t hi = bf16x2_bits(to_bf16x2(v2, v3));
      *reinterpret_cast<uint2*>(dst + n0) = make_uint2(lo, hi);
    }
  }
}

// fp32 variant: one thread per (token, output pair), plain fp32 FMA dot
// products in index order.
__global__ __launch_bounds__(256)
void append_f32_kernel(const float* __restrict__ x, int D, int ntok, int n_new,
                       const float* __restrict__ w_dkv, const float* __restrict__ w_kr, int d_c,
                       int W, const int* __restrict__ pos, float* __restrict__ cache, int cap,
                       int off, RopeSpec rope) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int pairs = W / 2;
  if (idx >= (int64_t)ntok * pairs) return;
  const int tok = (int)(idx / pairs), pr = (int)(idx - (int64_t)tok * pairs);
  const int n = 2 * pr;
  const float* w0 = n < d_c ? w_dkv + (int64_t)n * D : w_kr + (int64_t)(n - d_c) * D;
  const float* w1 = w0 + D;
  const float* xr = x + (int64_t)tok * D;
  float a0 = 0.f, a1 = 0.f;
  for (int k = 0; k < D; ++k) {
    a0 = fmaf(xr[k], w0[k], a0);
    a1 = fmaf(xr[k], w1[k], a1);
  }
  const int b = tok / n_new, i = tok - b * n_new;
  if (n >= d_c) {
    const double ang = rope_angle((n - d_c) >> 1, pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], rope);
    const float c = (float)cos(ang), s = (float)sin(ang);
    const float r0 = fmaf(a0, c, -(a1 * s)), r1 = fmaf(a0, s, a1 * c);
    a0 = r0; a1 = r1;
  }
  float* dst = cache + ((int64_t)b * cap + off + i) * W + n;
  dst[0] = a0;
  dst[1] = a1;
}

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s) {
  const int ntok = a.batch * a.n_new;
  const dim3 grid((ntok + 31) / 32), block(64);
  const u16* x = (const u16*)a.x;
  const u16* wd = (const u16*)a.w_dkv;
  const u16* wk = (const u16*)a.w_kr;
  u16* c = (u16*)a.cache;
  switch ((a.d_c + a.d_r) / 32) {
    case 3: append_bf16_kernel<3><<<grid, block, 0, s>>>(x, a.d_model, ntok, a.n_new, wd, wk, a.d_c, a.pos, c, a.cap, a.off, a.rope); break;
    case 5: append_bf16_kernel<5><<<grid, block, 0, s>>>(x, a.d_model, ntok, a.n_new, wd, wk, a.d_c, a.pos, c, a.cap, a.off, a.rope); break;
    case 7: append_bf16_kernel<7><<<grid, block, 0, s>>>(x, a.d_model, ntok, a.n_new, wd, wk, a.d_c, a.pos, c, a.cap, a.off, a.rope); break;
    case 9: append_bf16_kernel<9><<<grid, block, 0, s>>>(x, a.d_model, ntok, a.n_new, wd, wk, a.d_c, a.pos, c, a.cap, a.off, a.rope); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append_f32(const AppendArgs& a, hipStream_t s) {
  const int ntok = a.batch * a.n_new;
  const int W = a.d_c + a.d_r;
  const int64_t work = (int64_t)ntok * (W / 2);
  const dim3 grid((unsigned)((work + 255) / 256)), block(256);
  append_f32_kernel<<<grid, block, 0, s>>>((const float*)a.x, a.d_model, ntok, a.n_new,
                                           (const float*)a.w_dkv, (const float*)a.w_kr, a.d_c, W,
                                           a.pos, (float*)a.cache, a.cap, a.off, a.rope);
  return hipGetLastError();
}

}  // namespace mla
