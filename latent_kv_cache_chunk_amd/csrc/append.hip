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

// One workgroup computes 32 tokens x one block of 32 outputs with
// bf16 MFMA 32x32x16 and fp32 accumulation; a launch has (tokens / 32) x
// ((d_c + d_r) / 32) workgroups, enough to fill the chip at one chunk.  The
// four wavefronts split the reduction over d_model (a quarter each, loads
// issued eight k-steps ahead) and their fp32 partial sums are added in LDS, in
// a fixed order.  The product is formed transposed, C^T[n][token] = sum_k
// W[n][k] x[token][k]: weight rows (n) are the A operand, read from global
// memory (the whole [W_DKV; W_KR] is 688 KB at D = 1536, d_c = 192, and stays
// in L2), hidden states are the B operand.  In the epilogue each thread owns
// four consecutive outputs of one token, so the RoPE pairs are thread-local
// and the store is 8 bytes.
template <int NB>
__global__ __launch_bounds__(256)
void append_bf16_kernel(const u16* __restrict__ x, int D, int ntok, int n_new,
                        const u16* __restrict__ w_dkv, const u16* __restrict__ w_kr, int d_c,
                        const int* __restrict__ pos, u16* __restrict__ cache, int cap, int off,
                        RopeSpec rope) {
  constexpr int W = NB * 32;
  constexpr int UNROLL = 8;
  __shared__ float part[4][32][32 + 4];     // per-wave partial sums [token][n - n_base]

  // Workgroup id -> (token block tb, output block nb) so that the output
  // blocks of one token block get ids that are equal mod 8: workgroups are
  // dealt to the eight XCDs round robin, so they share that token block's
  // hidden states in one L2 (id = 8*NB*(tb/8) + 8*nb + tb%8).
  const int id = blockIdx.x;
  const int nb = (id >> 3) % NB, tb = (id / (8 * NB)) * 8 + (id & 7);
  if (tb * 32 >= ntok) return;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok0 = tb * 32;
  const int n_base = nb * 32;
  const int my_tok = tok0 + (lane & 31);
  const bool tok_ok = my_tok < ntok;
  const int kq = D / 4;                                  // this wave's share of the reduction
  const int kbeg = wave * kq;
  const u16* xrow = x + (int64_t)(tok_ok ? my_tok : 0) * D + kbeg + half * 8;
  const int n = n_base + (lane & 31);
  const u16* wrow = (n < d_c ? w_dkv + (int64_t)n * D : w_kr + (int64_t)(n - d_c) * D) + kbeg + half * 8;

  f32x16 acc = {};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int ksteps = kq / 16;
  int k = 0;
  for (; k + UNROLL <= ksteps; k += UNROLL) {
    bf16x8 bx[UNROLL], aw[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      bx[u] = tok_ok ? *reinterpret_cast<const bf16x8*>(xrow + (k + u) * 16) : __builtin_bit_cast(bf16x8, zero);
      aw[u] = *reinterpret_cast<const bf16x8*>(wrow + (k + u) * 16);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc = mfma_32x32x16(aw[u], bx[u], acc);
  }
  for (; k < ksteps; ++k) {
    const bf16x8 bx = tok_ok ? *reinterpret_cast<const bf16x8*>(xrow + k * 16) : __builtin_bit_cast(bf16x8, zero);
    acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(wrow + k * 16), bx, acc);
  }
  // partial sums -> LDS: lane holds token (lane & 31), outputs n_base + 8g + 4*half + t
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(&part[wave][lane & 31][g * 8 + half * 4]) =
        f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  __syncthreads();

  // epilogue: thread = 4 consecutive outputs of one token (32 x 32 / 4 = 256 groups)
  const int t = tid >> 3, n0 = (tid & 7) * 4;
  const int tok = tok0 + t;
  if (tok >= ntok) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(&part[0][t][n0]);
#pragma unroll
  for (int w2 = 1; w2 < 4; ++w2) v += *reinterpret_cast<const f32x4*>(&part[w2][t][n0]);
  const int b = tok / n_new, i = tok - b * n_new;
  const int nn = n_base + n0;
  if (nn >= d_c) {                                   // positional key: rotate the two pairs
    const int pt = pos[3 * i], ph = pos[3 * i + 1], pw = pos[3 * i + 2];
    const int pair = (nn - d_c) >> 1;
    const double a0 = rope_angle(pair, pt, ph, pw, rope);
    const double a1 = rope_angle(pair + 1, pt, ph, pw, rope);
    const float c0 = (float)cos(a0), s0 = (float)sin(a0);
    const float c1 = (float)cos(a1), s1 = (float)sin(a1);
    const float r0 = fmaf(v[0], c0, -(v[1] * s0)), r1 = fmaf(v[0], s0, v[1] * c0);
    const float r2 = fmaf(v[2], c1, -(v[3] * s1)), r3 = fmaf(v[2], s1, v[3] * c1);
    v = f32x4{r0, r1, r2, r3};
  }
  u16* dst = cache + ((int64_t)b * cap + off + i) * W + nn;
  *reinterpret_cast<uint2*>(dst) = make_uint2(bf16x2_bits(to_bf16x2(v[0], v[1])), bf16x2_bits(to_bf16x2(v[2], v[3])));
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
  const int tblocks = (ntok + 31) / 32;
  const int nbk = (a.d_c + a.d_r) / 32;
  const dim3 grid((unsigned)(((tblocks + 7) / 8) * 8 * nbk)), block(256);   // see the id mapping in the kernel
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
