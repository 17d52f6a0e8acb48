// Fused chunk attention over the latent cache.
//
// For every row r = (batch, head, query) of the current chunk and every
// visible key j (all cached chunks plus the chunk itself -- chunk-causal,
// bidirectional inside the chunk; VideoMLA atlas.scime.ai summary, first
// paragraph) the score is the dot product of the absorbed query q~_r with the
// cached row [c_j || k_R,j]; the kernel keeps an online base-2 softmax
// (running max m, running sum l) and accumulates L_r = sum_j p_rj c_j in fp32.
// Because every head reads the same latent rows (VideoMLA arXiv abstract: one
// latent and one positional key shared by all heads), a workgroup packs 256
// rows of any heads and streams each key tile through LDS once for all of them.
//
// MFMA formulation (bf16 32x32x16, fp32 accumulate), per wavefront of 64 rows:
//   S^T[key][row]  = K_tile[key][:] . q~[row][:]     A = key rows (LDS),
//                                                    B = q~ rows (registers)
//   O^T[c][row]   += V^T[c][key] . P^T[key][row]     A = transposed latent (LDS),
//                                                    B = P straight from S^T
// With keys on the MFMA rows, one lane holds 16 keys of one row, so the row
// max and row sum are lane-local plus one exchange with lane^32.  The S^T
// accumulator of lane-half h holds keys {8g + 4h + t}; the PV k-step reads
// those registers directly, so the transposed latent copy in LDS stores each
// 16-key group in the matching order {0-3, 8-11, 4-7, 12-15}.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Position of key k (0..15 inside a 16-key group) in the transposed copy.
__device__ inline int vperm16(int k) { return ((k & 4) << 1) | ((k >> 3) << 2) | (k & 3); }

template <int DC>
__global__ __launch_bounds__(256, 1)
void attend_bf16_kernel(const u16* __restrict__ cache, int64_t cache_bstride, int n_k,
                        const u16* __restrict__ qt, int rows_pad_b, int rb_per_b,
                        float* __restrict__ part_L, float* __restrict__ part_ml,
                        int T, int64_t U, int G) {
  constexpr int W = DC + 32;        // cached row width (elements)
  constexpr int KS = W / 16;        // k-steps of the score product
  constexpr int CB = DC / 32;       // 32-wide latent column blocks of O^T
  constexpr int BN = kKeyTile;      // 64 keys per tile
  constexpr int KROW = W + 8;       // padded LDS row of the key tile (conflict-free b128 reads)
  constexpr int VROW = BN + 8;      // padded LDS row of the transposed latent
  constexpr int NCH = W / 8;        // 16-byte chunks per cached row
  constexpr int VCH = DC / 8;       // chunks holding the latent c
  constexpr int STAGE_IT = BN * NCH / 256;
  static_assert(BN * NCH % 256 == 0, "tile chunks must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) u16 sK[BN * KROW];
  __shared__ __attribute__((aligned(16))) u16 sV[DC * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int64_t w = blockIdx.x;
  int64_t u = unit_begin(w, U, G);
  const int64_t u_end = unit_begin(w + 1, U, G);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  bool first_seg = true;

  while (u < u_end) {
    const int64_t rb = u / T;
    const int t0 = (int)(u - rb * T);
    const int t1 = (int)min<int64_t>((int64_t)T, (int64_t)t0 + (u_end - u));
    const int b = (int)(rb / rb_per_b);
    const int rbl = (int)(rb - (int64_t)b * rb_per_b);
    const u16* cb_base = cache + (int64_t)b * cache_bstride;

    // Absorbed queries of this wave's two 32-row blocks, as MFMA B operands.
    bf16x8 qf[2][KS];
    {
      const int64_t row0 = (int64_t)b * rows_pad_b + (int64_t)rbl * kRowsPerBlock + wave * 64;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const u16* qrow = qt + (row0 + qb * 32 + (lane & 31)) * W + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
      }
    }

    f32x16 oacc[2][CB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] = f32x16{};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

#pragma unroll 1
    for (int t = t0; t < t1; ++t) {
      const int key0 = t * BN;
      __syncthreads();  // every wave is done with the previous tile
      // ---- stage the key tile: row layout for scores, transposed latent for P.V
#pragma unroll
      for (int it = 0; it < STAGE_IT; ++it) {
        const int qidx = tid + 256 * it;
        const int key = qidx & (BN - 1), ch = qidx >> 6;
        const int gk = key0 + key;
        const bf16x8 v = gk < n_k
            ? *reinterpret_cast<const bf16x8*>(cb_base + (int64_t)gk * W + ch * 8)
            : __builtin_bit_cast(bf16x8, zero);
        *reinterpret_cast<bf16x8*>(sK + key * KROW + ch * 8) = v;
        if (ch < VCH) {
          const int vcol = (key & ~15) | vperm16(key & 15);
          const u32x4 words = __builtin_bit_cast(u32x4, v);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sV[(ch * 8 + e) * VROW + vcol] = (u16)(words[e >> 1] >> (16 * (e & 1)));
        }
      }
      __syncthreads();

      // ---- scores S^T: 2 key blocks x 2 row blocks
      f32x16 s[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) { s[qb][0] = f32x16{}; s[qb][1] = f32x16{}; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + (kb * 32 + (lane & 31)) * KROW + ks * 16 + half * 8);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[qb][kb] = mfma_32x32x16(a, qf[qb][ks], s[qb][kb]);
        }
      }

      // ---- online softmax (base 2; the scale and log2(e) are folded into q~)
      const bool tail = key0 + BN > n_k;
      bf16x8 pb[2][2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (tail) {
              const int key = key0 + kb * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
              if (key >= n_k) s[qb][kb][v] = -INFINITY;
            }
            mx = fmaxf(mx, s[qb][kb][v]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx);
        if (m_new > m_run[qb]) {
          const float alpha = exp2f(m_run[qb] - m_new);
          l_run[qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[qb][cb] *= alpha;
          m_run[qb] = m_new;
        }
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = exp2f(s[qb][kb][v] - m_new);
            s[qb][kb][v] = p;
            lsum += p;
          }
        l_run[qb] += lsum;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            bf16x8 pv;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const bf16x2 two = to_bf16x2(s[qb][kb][part * 8 + e], s[qb][kb][part * 8 + e + 1]);
              pv[e] = two[0];
              pv[e + 1] = two[1];
            }
            pb[qb][kb][part] = pv;
          }
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                sV + (cb * 32 + (lane & 31)) * VROW + kb * 32 + part * 16 + half * 8);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) oacc[qb][cb] = mfma_32x32x16(a, pb[qb][kb][part], oacc[qb][cb]);
          }
      }
    }

    // ---- write this segment's partial softmax state
    const int64_t slot = 2 * w + (first_seg ? 0 : 1);
    first_seg = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
      const int rl = wave * 64 + qb * 32 + (lane & 31);
      float* Ld = part_L + (slot * kRowsPerBlock + rl) * DC;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = cb * 32 + g * 8 + half * 4;
          *reinterpret_cast<f32x4*>(Ld + c0) =
              f32x4{oacc[qb][cb][4 * g], oacc[qb][cb][4 * g + 1], oacc[qb][cb][4 * g + 2], oacc[qb][cb][4 * g + 3]};
        }
      if (half == 0) {
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 0] = m_run[qb];
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 1] = l_tot;
      }
    }
    u += (t1 - t0);
  }
}

// fp32 variant: 8 threads per row, 32 rows per workgroup, one workgroup
// sweeps all keys (no key partition).  Scores are reduced over the 8 threads
// with shuffles; the final L is written normalized into slot = row-block.
template <int DC>
__global__ __launch_bounds__(256)
void attend_f32_kernel(const float* __restrict__ cache, int64_t cache_bstride, int n_k,
                       const float* __restrict__ qt, int rows_pad_b, int rb_per_b,
                       float* __restrict__ part_L) {
  constexpr int W = DC + 32, BN = 32, QJ = W / 8, LJ = DC / 8;
  __shared__ float sK[BN * W];
  const int tid = threadIdx.x, rloc = tid >> 3, sub = tid & 7;
  const int blocks_per_b = rows_pad_b / 32;
  const int b = blockIdx.x / blocks_per_b;
  const int r = (blockIdx.x - b * blocks_per_b) * 32 + rloc;   // row within sample
  const float* qrow = qt + ((int64_t)b * rows_pad_b + r) * W;
  float qv[QJ], lacc[LJ];
#pragma unroll
  for (int j = 0; j < QJ; ++j) qv[j] = qrow[sub + 8 * j];
#pragma unroll
  for (int j = 0; j < LJ; ++j) lacc[j] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float* cbase = cache + (int64_t)b * cache_bstride;
  for (int key0 = 0; key0 < n_k; key0 += BN) {
    const int nk = min(BN, n_k - key0);
    __syncthreads();
    for (int e = tid; e < nk * W; e += 256) sK[e] = cbase[(int64_t)key0 * W + e];
    __syncthreads();
    for (int k = 0; k < nk; ++k) {
      const float* kr = sK + k * W;
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < QJ; ++j) d = fmaf(qv[j], kr[sub + 8 * j], d);
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      d += __shfl_xor(d, 4);
      const float m_new = fmaxf(m, d);
      const float alpha = exp2f(m - m_new);
      const float p = exp2f(d - m_new);
      l = l * alpha + p;
#pragma unroll
      for (int j = 0; j < LJ; ++j) lacc[j] = fmaf(p, kr[sub + 8 * j], lacc[j] * alpha);
      m = m_new;
    }
  }
  const int rb = b * rb_per_b + r / kRowsPerBlock;
  float* Ld = part_L + ((int64_t)rb * kRowsPerBlock + (r % kRowsPerBlock)) * DC;
  const float inv = 1.f / l;
#pragma unroll
  for (int j = 0; j < LJ; ++j) Ld[sub + 8 * j] = lacc[j] * inv;
}

hipError_t launch_attend_bf16(const Plan& p, const AttendArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const u16* cache = (const u16*)a.cache;
  const u16* qt = (const u16*)(ws + p.off_qt);
  float* L = (float*)(ws + p.off_L);
  float* ml = (float*)(ws + p.off_ml);
  const dim3 grid(p.G), block(256);
  switch (p.d_c) {
    case 64: attend_bf16_kernel<64><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G); break;
    case 128: attend_bf16_kernel<128><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G); break;
    case 192: attend_bf16_kernel<192><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G); break;
    case 256: attend_bf16_kernel<256><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend_f32(const Plan& p, const AttendArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const float* cache = (const float*)a.cache;
  const float* qt = (const float*)(ws + p.off_qt);
  float* L = (float*)(ws + p.off_L);
  const dim3 grid(p.B * (p.rows_pad_b / 32)), block(256);
  switch (p.d_c) {
    case 64: attend_f32_kernel<64><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L); break;
    case 128: attend_f32_kernel<128><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L); break;
    case 192: attend_f32_kernel<192><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L); break;
    case 256: attend_f32_kernel<256><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
