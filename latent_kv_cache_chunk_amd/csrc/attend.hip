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
//   S^T[key][row]  = K_tile[key][:] . q~[row][:]     A = key rows (LDS, b128),
//                                                    B = q~ rows (registers)
//   O^T[c][row]   += V^T[c][key] . P^T[key][row]     A = latent columns read
//                                                    transposed from the same
//                                                    LDS tile (ds_read_tr16_b64),
//                                                    B = P straight from S^T
// With keys on the MFMA rows, one lane holds 16 keys of one row, so the row
// max and row sum are lane-local plus one exchange with lane^32.  Lane-half h
// of the S^T accumulator holds keys {8g + 4h + t}; the transposed loads fetch
// exactly those keys for the P.V k-step, so P never moves between lanes.
//
// Staging: each 64-key tile is copied global -> LDS with direct-to-LDS 16-byte
// loads (no registers), one row per key padded to an odd number of 16-byte
// slots so the b128 reads of 16 consecutive rows hit distinct banks.  Two
// buffers: the next tile's loads are in flight while the current one is used.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0), others free

template <int DC>
struct AttendTile {
  static constexpr int W = DC + 32;          // cached row width (elements)
  static constexpr int NCH = W / 8;          // 16-byte chunks per cached row
  static constexpr int NSLOT = NCH + 1;      // plus one pad slot: stride = 4 * odd dwords
  static constexpr int ROWB = NSLOT * 16;    // LDS bytes per key row
  static constexpr int BN = kKeyTile;        // keys per tile
  static constexpr int TILEB = BN * ROWB;    // LDS bytes per tile buffer
  static constexpr int NINST = NSLOT;        // 64 lanes x 16 B per load: BN*NSLOT/64 loads per tile
  static constexpr int INST_PER_WAVE = (NINST + 3) / 4;
};

// Byte offsets (relative to the tile's first key row in global memory) of the
// direct-to-LDS loads this lane issues, one per load of its wave; LDS slot
// s = inst*64 + lane holds chunk s % NSLOT of key s / NSLOT (the pad slot
// re-reads the row's last chunk).
template <int DC>
__device__ inline void tile_offsets(int wave, int lane, int (&off)[AttendTile<DC>::INST_PER_WAVE]) {
  using L = AttendTile<DC>;
#pragma unroll
  for (int i = 0; i < L::INST_PER_WAVE; ++i) {
    const int inst = min(wave + 4 * i, L::NINST - 1);
    const int slot = inst * 64 + lane;
    const int key = slot / L::NSLOT;
    const int ch = min(slot - key * L::NSLOT, L::NCH - 1);
    off[i] = (key * L::W + ch * 8) * 2;
  }
}

// Enqueue the direct-to-LDS loads of key tile [key0, key0+64) into `tile`.
// In the last (partial) tile, keys past n_k re-read key n_k-1; their scores
// are masked.
template <int DC>
__device__ inline void issue_tile(const char* gbase, int key0, int n_k, char* tile, int wave,
                                  const int (&off)[AttendTile<DC>::INST_PER_WAVE]) {
  using L = AttendTile<DC>;
  const char* src0 = gbase + (int64_t)key0 * L::W * 2;
  const bool partial = key0 + L::BN > n_k;
#pragma unroll
  for (int i = 0; i < L::INST_PER_WAVE; ++i) {
    const int inst = wave + 4 * i;
    if (inst < L::NINST) {
      int o = off[i];
      if (partial) {
        const int key = o / (L::W * 2);
        const int kc = min(key, n_k - 1 - key0);
        o += (kc - key) * L::W * 2;
      }
      __builtin_amdgcn_global_load_lds(src0 + o, (lds_void*)(tile + inst * 1024), 16, 0, 0);
    }
  }
}

// Softmax state of one wavefront (64 rows as two 32-row MFMA blocks).
//
// The accumulators are never rescaled inside the key loop (VALU work on them
// would force them out of the accumulator registers).  Instead the reference
// max m of each row is fixed by the first 32-key block of a segment, and
// later scores may exceed it by up to `headroom` in log2 units (32 by
// default): p = 2^(s - m) then stays below 2^headroom, far inside the
// fp32/bf16 range, and the
// result is the same softmax (numerator and denominator share m).  If any row
// of the workgroup exceeds the headroom, the segment restarts in an exact
// two-pass mode: a max-only sweep, then accumulation against the true max.
template <int DC>
struct WaveState {
  static constexpr int KS = (DC + 32) / 16, CB = DC / 32;
  bf16x8 qf[2][KS];     // absorbed queries, MFMA B operands
  f32x16 oacc[2][CB];   // O^T accumulators (latent columns x rows)
  float m_ref[2];       // reference max (base 2), identical in lanes l and l^32
  float l_run[2];       // this lane's part of the running sum
};

enum class Pass { kSingle, kMax, kAccum };

// Scores of one 32-key block for both row blocks.
template <int DC>
__device__ __forceinline__ void block_scores(const WaveState<DC>& st, const char* kbase, f32x16 (&s)[2]) {
  constexpr int KS = WaveState<DC>::KS;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbase + ks * 32);
    s[0] = mfma_32x32x16(a, st.qf[0][ks], s[0]);
    s[1] = mfma_32x32x16(a, st.qf[1][ks], s[1]);
  }
}

// One 32-key block of a staged tile.  `n_valid` = keys of the block that
// exist (< 32 only in the last tile).  Returns true (kSingle only) if a row
// exceeded the headroom, in which case the state must be discarded.
template <int DC, Pass P>
__device__ __forceinline__ bool attend_block(WaveState<DC>& st, const char* tile_row0, int s_off, int v_off,
                                             int n_valid, int half, bool first_block, float headroom) {
  using L = AttendTile<DC>;
  constexpr int CB = WaveState<DC>::CB, ROWB = L::ROWB;
  f32x16 s[2];
  block_scores<DC>(st, tile_row0 + s_off, s);
  const int thr = n_valid - half * 4;   // value v is key (v>>2)*8 + (v&3) + 4*half of the block
  bool over = false;
  bf16x8 pb[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (n_valid < 32) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((v >> 2) * 8 + (v & 3) >= thr) s[qb][v] = -INFINITY;
    }
    if (P != Pass::kAccum) {
      float mx = s[qb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[qb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (P == Pass::kMax) {
        st.m_ref[qb] = fmaxf(st.m_ref[qb], mx);
        continue;
      }
      if (first_block) st.m_ref[qb] = mx;
      over |= mx > st.m_ref[qb] + headroom;
    }
    const float m = st.m_ref[qb];
    float lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(s[qb][v] - m);
      s[qb][v] = p;
      lsum += p;
    }
    st.l_run[qb] += lsum;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      bf16x8 pv;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 two = to_bf16x2(s[qb][part * 8 + e], s[qb][part * 8 + e + 1]);
        pv[e] = two[0];
        pv[e + 1] = two[1];
      }
      pb[qb][part] = pv;
    }
  }
  if (P == Pass::kMax) return false;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const char* vbase = tile_row0 + part * 16 * ROWB + v_off;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + cb * 64));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + 8 * ROWB + cb * 64));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      st.oacc[0][cb] = mfma_32x32x16(a, pb[0][part], st.oacc[0][cb]);
      st.oacc[1][cb] = mfma_32x32x16(a, pb[1][part], st.oacc[1][cb]);
    }
  }
  return over;
}

// Both 32-key blocks of the tile held in `tile`.
template <int DC, Pass P>
__device__ __forceinline__ bool attend_tile(WaveState<DC>& st, const char* tile, int key0, int n_k,
                                            int s_off, int v_off, int half, bool first_tile, float headroom) {
  using L = AttendTile<DC>;
  const int left = n_k - key0;
  bool over = false;
#pragma unroll 1
  for (int kb = 0; kb < 2; ++kb) {
    const int n_valid = min(32, left - kb * 32);
    if (n_valid > 0)
      over |= attend_block<DC, P>(st, tile + kb * 32 * L::ROWB, s_off, v_off, n_valid, half,
                                  first_tile && kb == 0, headroom);
  }
  return over;
}

// Sweep tiles [t0, t1) of one segment through the two LDS buffers.  Returns
// true (kSingle only, identical in every wave) if the segment must be redone.
template <int DC, Pass P>
__device__ __forceinline__ bool sweep(WaveState<DC>& st, char* sbuf0, char* sbuf1, const char* gbase,
                                      int t0, int t1, int n_k, int wave, const int (&goff)[AttendTile<DC>::INST_PER_WAVE], int s_off, int v_off,
                                      int half, float headroom) {
  using L = AttendTile<DC>;
  constexpr int BN = L::BN;
  issue_tile<DC>(gbase, t0 * BN, n_k, sbuf0, wave, goff);
  wait_vmcnt0();
  __syncthreads();
#pragma unroll 1
  for (int t = t0; t < t1; t += 2) {
    if (t + 1 < t1) issue_tile<DC>(gbase, (t + 1) * BN, n_k, sbuf1, wave, goff);
    bool over = attend_tile<DC, P>(st, sbuf0, t * BN, n_k, s_off, v_off, half, t == t0, headroom);
    wait_vmcnt0();
    if (P == Pass::kSingle) {
      if (__syncthreads_or(over)) return true;
    } else {
      __syncthreads();
    }
    if (t + 1 >= t1) break;
    if (t + 2 < t1) issue_tile<DC>(gbase, (t + 2) * BN, n_k, sbuf0, wave, goff);
    over = attend_tile<DC, P>(st, sbuf1, (t + 1) * BN, n_k, s_off, v_off, half, false, headroom);
    wait_vmcnt0();
    if (P == Pass::kSingle) {
      if (__syncthreads_or(over)) return true;
    } else {
      __syncthreads();
    }
  }
  return false;
}

template <int DC>
__device__ __forceinline__ void reset_acc(WaveState<DC>& st) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int cb = 0; cb < WaveState<DC>::CB; ++cb) st.oacc[qb][cb] = f32x16{};
    st.l_run[qb] = 0.f;
  }
}

template <int DC>
__global__ __launch_bounds__(256, 1)
void attend_bf16_kernel(const u16* __restrict__ cache, int64_t cache_bstride, int n_k,
                        const u16* __restrict__ qt, int rows_pad_b, int rb_per_b,
                        float* __restrict__ part_L, float* __restrict__ part_ml,
                        int T, int64_t U, int G, float headroom) {
  using L = AttendTile<DC>;
  constexpr int W = L::W, KS = WaveState<DC>::KS, CB = WaveState<DC>::CB, ROWB = L::ROWB;

  // Two distinct buffers (not offsets into one array) so that the LDS reads
  // of one tile are not ordered behind the in-flight direct loads of the next.
  __shared__ __attribute__((aligned(1024))) char sbuf0[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char sbuf1[L::TILEB];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int goff[L::INST_PER_WAVE];
  tile_offsets<DC>(wave, lane, goff);
  // per-lane LDS offsets: b128 score operand, transposed latent operand
  const int s_off = (lane & 31) * ROWB + half * 16;
  const int g = lane >> 4, j = lane & 15;
  const int v_off = ((g >> 1) * 4 + (j >> 2)) * ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;

  const int64_t w = blockIdx.x;
  int64_t u = unit_begin(w, U, G);
  const int64_t u_end = unit_begin(w + 1, U, G);
  bool first_seg = true;
  WaveState<DC> st;

  while (u < u_end) {
    const int64_t rb = u / T;
    const int t0 = (int)(u - rb * T);
    const int t1 = (int)min<int64_t>((int64_t)T, (int64_t)t0 + (u_end - u));
    const int b = (int)(rb / rb_per_b);
    const int rbl = (int)(rb - (int64_t)b * rb_per_b);
    const char* gbase = reinterpret_cast<const char*>(cache + (int64_t)b * cache_bstride);

    {
      const int64_t row0 = (int64_t)b * rows_pad_b + (int64_t)rbl * kRowsPerBlock + wave * 64;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const u16* qrow = qt + (row0 + qb * 32 + (lane & 31)) * W + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) st.qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
      }
    }
    reset_acc<DC>(st);
    st.m_ref[0] = st.m_ref[1] = -INFINITY;
    if (sweep<DC, Pass::kSingle>(st, sbuf0, sbuf1, gbase, t0, t1, n_k, wave, goff, s_off, v_off, half, headroom)) {
      // A score exceeded the first block's max by more than the headroom:
      // exact two-pass evaluation of this segment.
      st.m_ref[0] = st.m_ref[1] = -INFINITY;
      sweep<DC, Pass::kMax>(st, sbuf0, sbuf1, gbase, t0, t1, n_k, wave, goff, s_off, v_off, half, headroom);
      reset_acc<DC>(st);
      sweep<DC, Pass::kAccum>(st, sbuf0, sbuf1, gbase, t0, t1, n_k, wave, goff, s_off, v_off, half, headroom);
    }

    // ---- write this segment's partial softmax state
    const int64_t slot = 2 * w + (first_seg ? 0 : 1);
    first_seg = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32);
      const int rl = wave * 64 + qb * 32 + (lane & 31);
      float* Ld = part_L + (slot * kRowsPerBlock + rl) * DC;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int c0 = cb * 32 + gg * 8 + half * 4;
          *reinterpret_cast<f32x4*>(Ld + c0) = f32x4{st.oacc[qb][cb][4 * gg], st.oacc[qb][cb][4 * gg + 1],
                                                     st.oacc[qb][cb][4 * gg + 2], st.oacc[qb][cb][4 * gg + 3]};
        }
      if (half == 0) {
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 0] = st.m_ref[qb];
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
    case 64: attend_bf16_kernel<64><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom); break;
    case 128: attend_bf16_kernel<128><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom); break;
    case 192: attend_bf16_kernel<192><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom); break;
    case 256: attend_bf16_kernel<256><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom); break;
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
