// Value up-projection with the merge of partial softmax states:
//   L[row]   = sum_s 2^(m_s - M) L_s[row] / sum_s 2^(m_s - M) l_s[row]
//   out[b,i,h,:] = W_UV[h] L[row]             (row = h*n_q + i of sample b)
// The per-head W_UV is applied after attention (multi-head latent attention,
// DeepSeek-V2, listed under "Builds on" on the VideoMLA pages), so values are
// never materialised per head.  L stays fp32 until this product: it is split
// as L = hi + lo with hi, lo in bf16 and both halves go through bf16 MFMA, which
// keeps ~16 significant bits of L.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

typedef __attribute__((address_space(3))) void lds_void;

// Slot permutation of a staged W_UV row (NP 16-byte pieces).  With 16 lanes
// reading one piece of 16 consecutive rows: a 128-byte row offset mod 256
// (NP = 8, 24) puts even and odd rows in opposite bank halves, so eight
// distinct values for each pair of rows suffice; a row stride that is a
// multiple of 256 bytes (NP = 16, 32) needs sixteen.
template <int NP>
__device__ inline int wuv_swizzle(int row) {
  static_assert(NP % 8 == 0, "whole groups of eight pieces");
  if constexpr ((NP * 16) % 256 == 0) return row & 15;
  else return (row >> 1) & 7;
}

// Two wavefronts per SIMD for d_c <= 192 (the merge is latency-bound); d_c =
// 256 needs the full register file for its 128 merged channels per lane.
template <int DC, bool OUT_F32>
__global__ __launch_bounds__(256, DC <= 192 ? 2 : 1)
void upproj_bf16_kernel(const float* __restrict__ part_L, const float* __restrict__ part_ml,
                        const int64_t* __restrict__ units_ws, const PartitionHeader* __restrict__ hdr,
                        int T, int rb_per_b, int n_q, int H, const u16* __restrict__ w_uv,
                        void* __restrict__ out) {
  constexpr int DH = 128, KSTEPS = DC / 16;
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5;
  const int i = blockIdx.y * 128 + wave * 32 + (lane & 31);
  const bool ok = i < n_q;
  const bool active = blockIdx.y * 128 + wave * 32 < n_q;   // some real row in this wavefront

  const int r = h * n_q + (ok ? i : 0);
  const int64_t rb = (int64_t)b * rb_per_b + r / kRowsPerBlock;
  const int rl = r % kRowsPerBlock;

  // The attention step's partition; owners of this row-block's first
  // key-tile unit and of its last unit, whose segments are merged.
  const PartitionHeader ph = *hdr;
  const int64_t U = ph.U, G = ph.G;
  const int64_t* units = ph.per_block_units ? units_ws : nullptr;
  const int64_t u_first = rb_first_tile_unit(units, T, rb), u_last = rb_first_unit(units, T, rb + 1) - 1;
  const int64_t wa = unit_owner(u_first, U, G), wb = unit_owner(u_last, U, G);

  // W_UV[h] (DH rows of DC bf16) staged once per workgroup by direct-to-LDS
  // loads, issued after the partition lookups (whose waits would otherwise
  // wait for them too) and before the partial states, so that they land
  // while those load.
  // Rows are not padded (a direct load fills 64 consecutive 16-byte slots);
  // 16-byte piece p of row r sits in slot p ^ wuv_swizzle(r) of its row, which
  // keeps the b128 operand reads (16 lanes = 16 consecutive rows, one piece)
  // on distinct banks.
  constexpr int NP = DC / 8;                      // 16-byte pieces per row
  constexpr int WROW = DC * 2;
  __shared__ __attribute__((aligned(16))) char wsh[DH * WROW];
  {
    const char* wsrc = reinterpret_cast<const char*>(w_uv + (int64_t)h * DH * DC);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int k = 0; k < DH * NP / 256; ++k) {    // 64-slot loads of this wavefront
      const int slot0 = (wave_u + 4 * k) * 64;
      const int slot = slot0 + lane, row = slot / NP, pp = slot - row * NP;
      const int piece = pp ^ wuv_swizzle<NP>(row);
      __builtin_amdgcn_global_load_lds(wsrc + (row * NP + piece) * 16, (lds_void*)(wsh + slot0 * 16), 16, 0, 0);
    }
  }

  // L of this lane's row and columns {ks*16 + half*8 + e}, merged over the
  // segments in one pass with a running max M: what is summed so far is
  // rescaled by 2^(M_old - M_new) when a segment raises it.  A segment with
  // no visible key of the row has m = -inf and weight 0.  At d_c >= 192 the
  // segments go two at a time, both segments' loads in flight together (still
  // two wavefronts per SIMD at d_c = 192; the narrower widths would lose a
  // wavefront per SIMD to it), which halves the serial round trips of rows
  // with many segments (about ten per row for a short query shard); an odd
  // last segment goes alone.  The update runs segment by segment in
  // workgroup order either way.
  float M = -INFINITY, lsum = 0.f;
  float lc[KSTEPS][8];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) lc[ks][e] = 0.f;
  auto merge = [&](const auto& segs_ml, const auto& x, int nseg) {
#pragma unroll
    for (int sg = 0; sg < nseg; ++sg) {
      const float m_w = segs_ml[sg][0], l_w = segs_ml[sg][1];
      const float m_new = fmaxf(M, m_w);
      const float keep = M == -INFINITY ? 0.f : exp2f(M - m_new);
      const float wgt = m_w == -INFINITY ? 0.f : exp2f(m_w - m_new);
      M = m_new;
      lsum = fmaf(lsum, keep, wgt * l_w);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lc[ks][e] = fmaf(wgt, x[sg][ks][0][e], lc[ks][e] * keep);
          lc[ks][4 + e] = fmaf(wgt, x[sg][ks][1][e], lc[ks][4 + e] * keep);
        }
    }
  };
  auto load = [&](int64_t w, float (&ml)[2], f32x4 (&x)[KSTEPS][2]) {
    const int64_t sl = seg_slot(w, rb);
    ml[0] = part_ml[(sl * kRowsPerBlock + rl) * 2];
    ml[1] = part_ml[(sl * kRowsPerBlock + rl) * 2 + 1];
    const float* src = part_L + part_L_index(sl, rl, half * 8, DC);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      x[ks][0] = *reinterpret_cast<const f32x4*>(src + ks * 512);         // channels ks*16 + half*8 + 0..3
      x[ks][1] = *reinterpret_cast<const f32x4*>(src + ks * 512 + 128);   // channels ks*16 + half*8 + 4..7
    }
  };
  int64_t w = active ? wa : wb + 1;
  if constexpr (DC >= 192) {
#pragma unroll 1
    for (; w + 1 <= wb; w += 2) {
      float ml[2][2];
      f32x4 x[2][KSTEPS][2];
      load(w, ml[0], x[0]);
      load(w + 1, ml[1], x[1]);
      merge(ml, x, 2);
    }
  }
#pragma unroll 1
  for (; w <= wb; ++w) {
    float ml[1][2];
    f32x4 x[1][KSTEPS][2];
    load(w, ml[0], x[0]);
    merge(ml, x, 1);
  }
  const float inv_l = 1.f / lsum;
  __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0): this wavefront's W_UV loads have landed
  __syncthreads();         // W_UV staged
  if (!active) return;     // no barriers follow

  f32x16 acc[DH / 32];
#pragma unroll
  for (int db = 0; db < DH / 32; ++db) acc[db] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int c0 = ks * 16 + half * 8;
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float v0 = ok ? lc[ks][e] * inv_l : 0.f, v1 = ok ? lc[ks][e + 1] * inv_l : 0.f;
      const bf16x2 h2 = to_bf16x2(v0, v1);
      const bf16x2 l2 = to_bf16x2(v0 - (float)h2[0], v1 - (float)h2[1]);
      hi[e] = h2[0]; hi[e + 1] = h2[1]; lo[e] = l2[0]; lo[e + 1] = l2[1];
    }
#pragma unroll
    for (int db = 0; db < DH / 32; ++db) {
      const int wr = db * 32 + (lane & 31);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wsh + wr * WROW + ((c0 / 8) ^ wuv_swizzle<NP>(wr)) * 16);
      acc[db] = mfma_32x32x16(a, hi, acc[db]);
      acc[db] = mfma_32x32x16(a, lo, acc[db]);
    }
  }
  if (!ok) return;
  const int64_t orow = (((int64_t)b * n_q + i) * H + h) * DH;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = db * 32 + g * 8 + half * 4;
      if (OUT_F32) {
        *reinterpret_cast<f32x4*>((float*)out + orow + d0) =
            f32x4{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
      } else {
        const uint32_t lo2 = bf16x2_bits(to_bf16x2(acc[db][4 * g], acc[db][4 * g + 1]));
        const uint32_t hi2 = bf16x2_bits(to_bf16x2(acc[db][4 * g + 2], acc[db][4 * g + 3]));
        *reinterpret_cast<uint2*>((u16*)out + orow + d0) = make_uint2(lo2, hi2);
      }
    }
}

// fp32 variant: thread per output element; L comes normalized from slot rb.
template <bool OUT_F32>
__global__ __launch_bounds__(256)
void upproj_f32_kernel(const float* __restrict__ part_L, int B, int rb_per_b, int n_q, int H, int DC,
                       const float* __restrict__ w_uv, void* __restrict__ out) {
  constexpr int DH = 128;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * n_q * H * DH;
  if (idx >= total) return;
  const int d = (int)(idx % DH);
  const int64_t bih = idx / DH;
  const int h = (int)(bih % H);
  const int64_t bi = bih / H;
  const int i = (int)(bi % n_q), b = (int)(bi / n_q);
  const int r = h * n_q + i;
  const int64_t rb = (int64_t)b * rb_per_b + r / kRowsPerBlock;
  const float* L = part_L + (rb * kRowsPerBlock + r % kRowsPerBlock) * DC;
  const float* wv = w_uv + ((int64_t)h * DH + d) * DC;
  float acc = 0.f;
  for (int c = 0; c < DC; ++c) acc = fmaf(wv[c], L[c], acc);
  if (OUT_F32) ((float*)out)[idx] = acc;
  else ((u16*)out)[idx] = __builtin_bit_cast(u16, (__bf16)acc);
}

hipError_t launch_upproj_bf16(const Plan& p, const UpprojArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const float* L = (const float*)(ws + p.off_L);
  const float* ml = (const float*)(ws + p.off_ml);
  const int64_t* units = (const int64_t*)(ws + p.off_units);
  const PartitionHeader* hdr = (const PartitionHeader*)(ws + p.off_hdr);
  const u16* wv = (const u16*)a.w_uv;
  const dim3 grid(p.B * p.H, (p.n_q + 127) / 128), block(256);
#define MLA_UPPROJ(DCV)                                                                                       \
  if (a.out_f32) upproj_bf16_kernel<DCV, true><<<grid, block, 0, s>>>(L, ml, units, hdr, p.T, p.rb_per_b, p.n_q, p.H, wv, a.out); \
  else upproj_bf16_kernel<DCV, false><<<grid, block, 0, s>>>(L, ml, units, hdr, p.T, p.rb_per_b, p.n_q, p.H, wv, a.out);
  switch (p.d_c) {
    case 64: MLA_UPPROJ(64) break;
    case 128: MLA_UPPROJ(128) break;
    case 192: MLA_UPPROJ(192) break;
    case 256: MLA_UPPROJ(256) break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_UPPROJ
  return hipGetLastError();
}

hipError_t launch_upproj_f32(const Plan& p, const UpprojArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const float* L = (const float*)(ws + p.off_L);
  const int64_t total = (int64_t)p.B * p.n_q * p.H * 128;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (a.out_f32)
    upproj_f32_kernel<true><<<grid, block, 0, s>>>(L, p.B, p.rb_per_b, p.n_q, p.H, p.d_c, (const float*)a.w_uv, a.out);
  else
    upproj_f32_kernel<false><<<grid, block, 0, s>>>(L, p.B, p.rb_per_b, p.n_q, p.H, p.d_c, (const float*)a.w_uv, a.out);
  return hipGetLastError();
}

}  // namespace mla
