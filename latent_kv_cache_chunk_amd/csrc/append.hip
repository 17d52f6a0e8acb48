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

// One workgroup computes 32 tokens x one block of 32 outputs with bf16 MFMA
// 32x32x16 and fp32 accumulation; a launch has (tokens / 32) x ((d_c + d_r) /
// 32) workgroups, enough to fill the chip at one chunk.  The product is formed
// transposed, C^T[n][token] = sum_k W[n][k] x[token][k]: weight rows (n) are
// the A operand (the whole [W_DKV; W_KR] is 688 KB at D = 1536, d_c = 192, and
// stays in L2), hidden states the B operand.
//
// d_model is cut into 64-wide chunks dealt round robin to the four
// wavefronts; their fp32 partial sums are added in LDS in a fixed order.  A
// chunk is 32 rows x 128 bytes of x and of W.  Global loads are row-major
// (eight lanes read one row's 128 bytes, so a load instruction covers eight
// whole cache lines), two chunks in flight in registers; each chunk then
// goes through the wavefront's own 8 KB of LDS, where 16-byte piece p of row r
// sits in slot p ^ (r & 7), and comes back in MFMA operand layout.  Both the
// row-major writes and the operand reads (eight rows per 128 bytes of banks)
// are conflict-free.  Which eight k of a 16-wide k-step a lane half holds does
// not change the sum: lane half h of k-step j holds piece 2j + h of the chunk,
// in A and B alike.
//
// In the epilogue each thread owns four consecutive outputs of one token, so
// the RoPE pairs are thread-local and the store is 8 bytes.
constexpr int kAppendChunk = 64;          // k per chunk
constexpr int kAppendRing = 2;            // chunks in flight per wavefront

struct AppendChunk {
  u32x4 x[4], w[4];                       // rows q*8 + lane/8, piece lane%8
};

template <int NB>
__global__ __launch_bounds__(256)
void append_bf16_kernel(const u16* __restrict__ x, int D, int ntok, int n_new,
                        const u16* __restrict__ w_dkv, const u16* __restrict__ w_kr, int d_c,
                        const int* __restrict__ pos, u16* __restrict__ cache, int cap, int off,
                        RopeSpec rope) {
  constexpr int W = NB * 32;
  __shared__ __attribute__((aligned(16))) char stage[4][2][32 * 128];   // [wave][x | w] chunk rows
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

  // The epilogue's rotation depends only on positions, so the workgroups of
  // the positional block evaluate it (fp64 angles, then cos and sin) before
  // their k loop: its latency then overlaps the loads of the CU's other
  // workgroups instead of extending this workgroup's tail.  Thread mapping as
  // in the epilogue (token tid / 8, outputs n_base + (tid % 8) * 4 .. + 3).
  float rc0 = 1.f, rs0 = 0.f, rc1 = 1.f, rs1 = 0.f;
  if (n_base + 32 > d_c) {
    const int et = threadIdx.x >> 3, enn = n_base + (threadIdx.x & 7) * 4;
    if (enn >= d_c) {
      const int ei = min(tok0 + et, ntok - 1) % n_new;
      const int pt = pos[3 * ei], ph = pos[3 * ei + 1], pw = pos[3 * ei + 2];
      const int pair = (enn - d_c) >> 1;
      const double a0 = rope_angle(pair, pt, ph, pw, rope);
      const double a1 = rope_angle(pair + 1, pt, ph, pw, rope);
      rc0 = (float)cos(a0); rs0 = (float)sin(a0);
      rc1 = (float)cos(a1); rs1 = (float)sin(a1);
    }
  }

  // global row pointers of this lane's four x rows and four W rows (row-major loads)
  const int lrow = lane >> 3, piece = lane & 7;
  const u16* xr[4];
  const u16* wr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tok = min(tok0 + q * 8 + lrow, ntok - 1);   // rows past the last token re-read it
    xr[q] = x + (int64_t)tok * D + piece * 8;
    const int n = n_base + q * 8 + lrow;
    wr[q] = (n < d_c ? w_dkv + (int64_t)n * D : w_kr + (int64_t)(n - d_c) * D) + piece * 8;
  }
  char* xs = stage[wave][0];
  char* ws = stage[wave][1];
  const int wslot = lrow * 128 + ((piece ^ lrow) * 16);            // row-major write slot (row & 7 == lrow)
  const int r = lane & 31;
  const int nchunks = D / kAppendChunk;
  const int mine = (nchunks - wave + 3) / 4;                       // chunks wave, wave + 4, ...

  // Chunk i of this wavefront (clamped to its last one: the prologue of a
  // wavefront with a single chunk loads it twice and uses it once).
  auto issue = [&](AppendChunk& ck, int i) {
    const int k0 = (wave + 4 * min(i, mine - 1)) * kAppendChunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ck.x[q] = *reinterpret_cast<const u32x4*>(xr[q] + k0);
      ck.w[q] = *reinterpret_cast<const u32x4*>(wr[q] + k0);
    }
  };
  f32x16 acc = {};
  auto consume = [&](const AppendChunk& ck) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<u32x4*>(xs + q * 1024 + wslot) = ck.x[q];
      *reinterpret_cast<u32x4*>(ws + q * 1024 + wslot) = ck.w[q];
    }
    // the wavefront's LDS accesses run in order; these only keep the
    // compiler from moving the operand reads above other lanes' writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    bf16x8 a[kAppendChunk / 16], b[kAppendChunk / 16];
#pragma unroll
    for (int j = 0; j < kAppendChunk / 16; ++j) {
      const int off_b = r * 128 + (((2 * j + half) ^ (r & 7)) * 16);
      a[j] = *reinterpret_cast<const bf16x8*>(ws + off_b);
      b[j] = *reinterpret_cast<const bf16x8*>(xs + off_b);
    }
#pragma unroll
    for (int j = 0; j < kAppendChunk / 16; ++j) acc = mfma_32x32x16(a[j], b[j], acc);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Two chunks in flight.  Every pass of the loop issues exactly two more (so
  // the wait before each chunk's first use is the same on every path); the
  // last two are consumed after it.
  if (mine > 0) {
    AppendChunk c0, c1;
    issue(c0, 0);
    issue(c1, 1);
    int i = 0;
#pragma unroll 1
    for (; i + kAppendRing < mine; i += kAppendRing) {
      consume(c0);
      issue(c0, i + 2);
      consume(c1);
      issue(c1, i + 3);
    }
    consume(c0);
    if (i + 1 < mine) consume(c1);
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
    const float c0 = rc0, s0 = rs0, c1 = rc1, s1 = rs1;
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
