// Standard multi-head attention over per-head keys and values.
//
// Two uses, both for comparison with the latent path of attend.hip:
//  * the dense per-head K/V cache that VideoMLA replaces (2 x H x d_h values
//    per token against d_c + d_r; atlas.scime.ai summary, "Key results"):
//      out[b,i,h] = sum_j softmax_j(scale * q[b,i,h] . k[b,j,h]) v[b,j,h];
//  * the non-absorbed form of multi-head latent attention (DeepSeek-V2,
//    listed under "Builds on" on the VideoMLA pages): K_h = [C W_UK[h]^T || K_R]
//    and V_h = C W_UV[h]^T are materialised from the latent cache once per
//    call, then the same attention runs with d_qk = d_h + d_r.
//
// The attention kernel has the wavefront roles of attend.hip: a workgroup
// owns 256 rows of one (batch, head), in four groups of 64 with a score
// wavefront (q in registers, S^T = K q^T by bf16 32x32x16 MFMA,
// p = 2^(qscale*s - m), P to LDS) and a value wavefront (O^T += V^T P^T, V^T
// read transposed from LDS) on each SIMD.  Keys and values are staged by
// direct-to-LDS loads in 64-key tiles, in separate double buffers: in step
// k the score side reads K of tile k while K of tile k+1 arrives, and the
// value side reads V of tile k-1 while V of tile k arrives, so two buffers
// of each serve where a combined [k || v] row would need three (which would
// not fit the LDS at 64 keys).  Partial softmax states per (workgroup, row
// block) are merged by mha_merge_kernel.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {
namespace mha {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0), others free

constexpr int kWaves = 8;          // wavefronts per workgroup
constexpr int kGroups = 4;         // row groups (score + value wavefront each)
constexpr int kGroupRows = 64;     // rows per group: two 32-row MFMA blocks
constexpr int kBN = 64;            // keys per tile: two 32-key MFMA blocks
constexpr int kDV = 128;           // value width (head_dim)

// LDS staging of one tensor's rows of a 64-key tile: rows padded by one
// 16-byte slot (odd stride in 16-byte units); one 64-lane direct-to-LDS
// load copies ROWS whole rows, the pad lane re-reading the row's last chunk.
template <int D>
struct Rows {
  static constexpr int NCH = D / 8;                 // 16-byte chunks of a row
  static constexpr int NSLOT = NCH + 1;
  static constexpr int ROWB = NSLOT * 16;           // LDS bytes per key
  static constexpr int BUF = kBN * ROWB;            // LDS bytes per tile
  static constexpr int ROWS = 64 / NSLOT;           // rows per load
  static constexpr int NLOAD = (kBN + ROWS - 1) / ROWS;
  static constexpr int PER_WAVE = (NLOAD + kGroups - 1) / kGroups;   // value wavefronts issue the loads
  static_assert(ROWS >= 1 && (NSLOT & 1), "a row fits one load, odd slot stride");
};

template <int DQK>
struct Tile {
  using K = Rows<DQK>;
  using V = Rows<kDV>;
  static constexpr int KS = DQK / 16;         // score k-steps
  static constexpr int CB = kDV / 32;         // 32-column blocks of O^T
  static constexpr int PBUF = kGroups * 2 * 2 * 2 * 64 * 16;   // P bytes of one tile (group, kb, qb, part, lane)
  static_assert(2 * K::BUF + 2 * V::BUF + 2 * PBUF <= 160 * 1024, "buffers exceed LDS");
};

// Per-lane slot of the direct-to-LDS copies of one tensor.
struct LaneCopy {
  uint32_t chunk;   // byte offset of the lane's chunk inside its row
  int row;          // row of the load the lane copies (>= ROWS: idle)
};

template <int D>
__device__ inline LaneCopy lane_copy(int lane) {
  using R = Rows<D>;
  LaneCopy lc;
  lc.row = lane / R::NSLOT;
  lc.chunk = (uint32_t)min(lane - lc.row * R::NSLOT, R::NCH - 1) * 16;
  return lc;
}

struct Ctx {
  __amdgpu_buffer_rsrc_t ksrc;   // buffer resource over the n_k keys of this (batch, head) in K
  __amdgpu_buffer_rsrc_t vsrc;   // and in V
  uint32_t krow, vrow;   // bytes between consecutive keys in K and V
  LaneCopy kc, vc;
  int n_k;
  int wave, lane, half, group;
  int s_off, v_off;      // LDS operand offsets inside a tile
};

// Enqueue this value wavefront's share of the direct-to-LDS loads of tile t
// of one tensor (the score wavefronts, each step's critical path, issue
// none): load ld copies rows [ld*ROWS, ld*ROWS + ROWS).  Keys past n_k
// re-read key n_k - 1 (their scores are masked).  Offsets are 32-bit: one
// (batch, head)'s keys span less than 4 GiB.  The copies are buffer loads to
// LDS: after a global load to LDS the compiler must assume the load may still
// touch LDS out of order, and every wait on this wavefront's own LDS reads
// became a wait for all of them.
template <int D>
__device__ inline void issue_rows(const Ctx& c, __amdgpu_buffer_rsrc_t src, uint32_t row_bytes, const LaneCopy& lc,
                                  int t, char* buf) {
  using R = Rows<D>;
#pragma unroll
  for (int i = 0; i < R::PER_WAVE; ++i) {
    const int ld = c.group + kGroups * i;
    if (ld < R::NLOAD) {
      const int row0 = ld * R::ROWS;
      const uint32_t key = (uint32_t)min(t * kBN + row0 + lc.row, c.n_k - 1);
      if (lc.row < R::ROWS && row0 + lc.row < kBN)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)(buf + row0 * R::ROWB), 16, key * row_bytes + lc.chunk,
                                                 0, 0, 0);
    }
  }
}

enum class Pass { kSingle, kMax, kAccum };

__device__ __forceinline__ int p_slot(int g, int kb, int qb, int part, int lane) {
  return ((((g * 2 + kb) * 2 + qb) * 2 + part) * 64 + lane) * 16;
}

__device__ __forceinline__ void mask_block(f32x16& s, int n_valid, int half) {
  const int thr = n_valid - half * 4;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if ((v >> 2) * 8 + (v & 3) >= thr) s[v] = -INFINITY;
}

__device__ __forceinline__ float block_max(const f32x16& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float b = fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]));
  const float c = fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11]));
  const float d = fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]));
  const float m = fmaxf(fmaxf(a, b), fmaxf(c, d));
  return fmaxf(m, __shfl_xor(m, 32));
}

template <int DQK>
struct ScoreState {
  bf16x8 qf[2][Tile<DQK>::KS];
  float qscale;          // softmax_scale * log2(e), applied to the fp32 scores
  float m_ref[2];        // reference max, scaled (log2 units)
  float l_run[2];
};

// Scores of tile t: S^T = K q^T for the two 32-key blocks and two 32-row
// blocks of the group, then p = 2^(qscale*s - m) to the P buffer as the
// B operand of the value product.
template <int DQK, Pass P>
__device__ __forceinline__ void score_tile(ScoreState<DQK>& st, const char* kbuf, char* pbuf, int t, bool first,
                                           const Ctx& c) {
  using L = Tile<DQK>;
  constexpr int KS = L::KS, PF = 4;
  // One stream of K operand reads over both blocks, each PF k-steps ahead of
  // its MFMAs (read g = block g / KS, k-step g % KS, in slot g % PF).
  bf16x8 a[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) a[i] = *reinterpret_cast<const bf16x8*>(kbuf + c.s_off + i * 32);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int g = kb * KS + ks, gn = g + PF;
      const bf16x8 cur = a[g % PF];
      if (gn < 2 * KS)
        a[g % PF] = *reinterpret_cast<const bf16x8*>(kbuf + (gn / KS) * 32 * L::K::ROWB + c.s_off + (gn % KS) * 32);
      s[0] = mfma_32x32x16(cur, st.qf[0][ks], s[0]);
      s[1] = mfma_32x32x16(cur, st.qf[1][ks], s[1]);
    }
    if (kb == 0) __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (kb * KS + ks + PF < 2 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    const int left = c.n_k - t * kBN - kb * 32;
    if (left < 32) {
      mask_block(s[0], left, c.half);
      mask_block(s[1], left, c.half);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (P == Pass::kMax) {
        st.m_ref[qb] = fmaxf(st.m_ref[qb], block_max(s[qb]) * st.qscale);
        continue;
      }
      if (P == Pass::kSingle && first && kb == 0) st.m_ref[qb] = block_max(s[qb]) * st.qscale;
      const float m = st.m_ref[qb];
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(s[qb][v], st.qscale, -m));
      float q[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) q[v] = p[2 * v] + p[2 * v + 1];
      st.l_run[qb] += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        bf16x8 pv;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 two = to_bf16x2(p[part * 8 + e], p[part * 8 + e + 1]);
          pv[e] = two[0];
          pv[e + 1] = two[1];
        }
        *reinterpret_cast<bf16x8*>(pbuf + p_slot(c.group, kb, qb, part, c.lane)) = pv;
      }
    }
  }
}

struct ValueState {
  f32x16 oacc[2][kDV / 32];
};

// O^T += V^T P^T for the tile's two 32-key blocks; V^T is read transposed
// from LDS (ds_read_tr16_b64), the key order inside each 16-key step
// matching the order in which the score wavefront stored P.
template <int DQK>
__device__ __forceinline__ void value_tile(ValueState& st, const char* vbuf, const char* pbuf, const Ctx& c) {
  using L = Tile<DQK>;
  constexpr int VR = L::V::ROWB;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const bf16x8 p0 = *reinterpret_cast<const bf16x8*>(pbuf + p_slot(c.group, kb, 0, part, c.lane));
      const bf16x8 p1 = *reinterpret_cast<const bf16x8*>(pbuf + p_slot(c.group, kb, 1, part, c.lane));
      const char* vb = vbuf + (kb * 32 + part * 16) * VR + c.v_off;
      bf16x8 av[L::CB];
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + cb * 64));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * VR + cb * 64));
        av[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) {
        st.oacc[0][cb] = mfma_32x32x16(av[cb], p0, st.oacc[0][cb]);
        st.oacc[1][cb] = mfma_32x32x16(av[cb], p1, st.oacc[1][cb]);
      }
      // the P reads and three column blocks' reads first, then two MFMAs and
      // the reads three column blocks ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (cb + 3 < L::CB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
}

// Step k of a sweep over tiles t0 .. t0+n-1: start K of tile k+1 and V of
// tile k; the score wavefront scores tile k (K buffer k % 2, P buffer k % 2),
// the value wavefront multiplies tile k-1 (V buffer (k-1) % 2, P buffer
// (k-1) % 2); wait; barrier.  Steps k = 0 .. n; true after step n.
template <int DQK, Pass P, bool SCORE, class State>
__device__ __forceinline__ bool sweep_step(State& st, int k, int n, int t0, char* kcur, char* knxt, char* vload,
                                           char* vprev, char* pcur, char* pprev, const Ctx& c) {
  if (!SCORE && k + 1 < n) issue_rows<DQK>(c, c.ksrc, c.krow, c.kc, t0 + k + 1, knxt);
  if (!SCORE && P != Pass::kMax && k < n) issue_rows<kDV>(c, c.vsrc, c.vrow, c.vc, t0 + k, vload);
  if constexpr (SCORE) {
    if (k < n) score_tile<DQK, P>(st, kcur, pcur, t0 + k, k == 0, c);
  } else {
    if (P != Pass::kMax && k >= 1) value_tile<DQK>(st, vprev, pprev, c);
  }
  wait_vmcnt0();
  __syncthreads();
  return k >= n;
}

template <int DQK, Pass P, bool SCORE, class State>
__device__ __forceinline__ void sweep(State& st, char* k0, char* k1, char* v0, char* v1, char* pb0, char* pb1,
                                      int t0, int t1, const Ctx& c) {
  const int n = t1 - t0;
  if (!SCORE) issue_rows<DQK>(c, c.ksrc, c.krow, c.kc, t0, k0);
  wait_vmcnt0();
  __syncthreads();
#pragma unroll 1
  for (int k = 0;; k += 2) {
    if (sweep_step<DQK, P, SCORE>(st, k, n, t0, k0, k1, v0, v1, pb0, pb1, c)) break;
    if (sweep_step<DQK, P, SCORE>(st, k + 1, n, t0, k1, k0, v1, v0, pb1, pb0, c)) break;
  }
}

struct Problem {
  const u16* q;          // queries [B*H][rows_pad_h][DQK], bf16, unscaled
  const u16* k;          // [B, cap, H, DQK], or [B, H, cap, DQK] when head_major
  const u16* v;          // [B, cap, H, kDV], or [B, H, cap, kDV] when head_major
  int64_t cap;
  bool head_major;
  int H, n_k, rows_pad_h, rb_per_bh, T;
  int64_t U;
  int G;
  float headroom;
  float qscale;          // softmax_scale * log2(e)
  float* part_L;         // [slots][256][kDV]
  float* part_ml;        // [slots][256][2]
};

// Row block rb = (b*H + h) * rb_per_bh + rbl; its units are rb*T .. rb*T + T - 1.
template <int DQK>
__device__ __forceinline__ void begin_segment(Ctx& c, const Problem& pr, int64_t rb) {
  const int64_t bh = rb / pr.rb_per_bh;
  const int b = (int)(bh / pr.H), h = (int)(bh - (int64_t)b * pr.H);
  // row (of DQK or kDV elements) of key 0 of this (batch, head)
  const int64_t tok0 = pr.head_major ? ((int64_t)b * pr.H + h) * pr.cap : (int64_t)b * pr.cap * pr.H + h;
  // bytes from key 0 to the end of key n_k - 1 (below 4 GiB; read unsigned)
  const uint32_t kbytes = (uint32_t)(pr.n_k - 1) * c.krow + DQK * 2, vbytes = (uint32_t)(pr.n_k - 1) * c.vrow + kDV * 2;
  c.ksrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(pr.k + tok0 * DQK), 0, (int)kbytes, 0x00020000);
  c.vsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(pr.v + tok0 * kDV), 0, (int)vbytes, 0x00020000);
}

template <int DQK, bool SCORE>
__device__ __forceinline__ void role(Ctx& c, const Problem& pr, int64_t w, char* k0, char* k1, char* v0, char* v1,
                                     char* pb0, char* pb1) {
  using L = Tile<DQK>;
  // segments last row block first (see the latent attention kernel): a range
  // that crosses a row-block boundary starts at key tile 0
  const int64_t u = unit_begin(w, pr.U, pr.G);
  int64_t u_end = unit_begin(w + 1, pr.U, pr.G);
  ScoreState<DQK> ss;
  ValueState vs;
  while (u < u_end) {
    const int64_t rb = (u_end - 1) / pr.T;
    const int64_t begin = max(u, rb * pr.T);
    const int t0 = (int)(begin - rb * pr.T);
    const int t1 = (int)(u_end - rb * pr.T);
    begin_segment<DQK>(c, pr, rb);
    const int64_t bh = rb / pr.rb_per_bh;
    const int rbl = (int)(rb - bh * pr.rb_per_bh);
    bool bad = false;
    if constexpr (SCORE) {
      const u16* qg = pr.q + (bh * pr.rows_pad_h + (int64_t)rbl * kRowsPerBlock + c.group * kGroupRows) * DQK;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const u16* qrow = qg + (int64_t)(qb * 32 + (c.lane & 31)) * DQK + c.half * 8;
#pragma unroll
        for (int ks = 0; ks < L::KS; ++ks) ss.qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
        ss.l_run[qb] = 0.f;
        ss.m_ref[qb] = -INFINITY;
      }
      ss.qscale = pr.qscale;
      sweep<DQK, Pass::kSingle, true>(ss, k0, k1, v0, v1, pb0, pb1, t0, t1, c);
      const float lim = __builtin_amdgcn_exp2f(pr.headroom);
      bad = !(ss.l_run[0] <= lim) || !(ss.l_run[1] <= lim);
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int cb = 0; cb < L::CB; ++cb) vs.oacc[qb][cb] = f32x16{};
      sweep<DQK, Pass::kSingle, false>(vs, k0, k1, v0, v1, pb0, pb1, t0, t1, c);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int cb = 0; cb < L::CB; ++cb)
#pragma unroll
          for (int v = 0; v < 16; ++v) bad |= !(fabsf(vs.oacc[qb][cb][v]) <= 3.0e38f);
    }
    if (__syncthreads_or(bad)) {
      // exact two-pass evaluation of this segment: the true max, then accumulation
      if constexpr (SCORE) {
        ss.m_ref[0] = ss.m_ref[1] = -INFINITY;
        sweep<DQK, Pass::kMax, true>(ss, k0, k1, v0, v1, pb0, pb1, t0, t1, c);
        ss.l_run[0] = ss.l_run[1] = 0.f;
        sweep<DQK, Pass::kAccum, true>(ss, k0, k1, v0, v1, pb0, pb1, t0, t1, c);
      } else {
        sweep<DQK, Pass::kMax, false>(vs, k0, k1, v0, v1, pb0, pb1, t0, t1, c);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int cb = 0; cb < L::CB; ++cb) vs.oacc[qb][cb] = f32x16{};
        sweep<DQK, Pass::kAccum, false>(vs, k0, k1, v0, v1, pb0, pb1, t0, t1, c);
      }
    }
    const int64_t slot = seg_slot(w, rb);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int rl = c.group * kGroupRows + qb * 32 + (c.lane & 31);
      if constexpr (SCORE) {
        const float l_tot = ss.l_run[qb] + __shfl_xor(ss.l_run[qb], 32);
        if (c.half == 0) {
          pr.part_ml[(slot * kRowsPerBlock + rl) * 2 + 0] = ss.m_ref[qb];
          pr.part_ml[(slot * kRowsPerBlock + rl) * 2 + 1] = l_tot;
        }
      } else {
        float* Ld = pr.part_L + (slot * kRowsPerBlock + rl) * kDV;
#pragma unroll
        for (int cb = 0; cb < L::CB; ++cb)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const int c0 = cb * 32 + gg * 8 + c.half * 4;
            *reinterpret_cast<f32x4*>(Ld + c0) = f32x4{vs.oacc[qb][cb][4 * gg], vs.oacc[qb][cb][4 * gg + 1],
                                                       vs.oacc[qb][cb][4 * gg + 2], vs.oacc[qb][cb][4 * gg + 3]};
          }
      }
    }
    u_end = begin;
  }
}

template <int DQK>
__global__ __launch_bounds__(kWaves * 64, 1)
void mha_attend_kernel(Problem pr) {
  using L = Tile<DQK>;
  __shared__ __attribute__((aligned(1024))) char kbuf0[L::K::BUF];
  __shared__ __attribute__((aligned(1024))) char kbuf1[L::K::BUF];
  __shared__ __attribute__((aligned(1024))) char vbuf0[L::V::BUF];
  __shared__ __attribute__((aligned(1024))) char vbuf1[L::V::BUF];
  __shared__ __attribute__((aligned(1024))) char pbuf0[L::PBUF];
  __shared__ __attribute__((aligned(1024))) char pbuf1[L::PBUF];
  Ctx c;
  c.n_k = pr.n_k;
  c.krow = (uint32_t)(pr.head_major ? 1 : pr.H) * DQK * 2;
  c.vrow = (uint32_t)(pr.head_major ? 1 : pr.H) * kDV * 2;
  c.lane = threadIdx.x & 63;
  c.half = c.lane >> 5;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = c.wave < kGroups;   // wavefronts w and w + 4 share a SIMD
  c.group = c.wave & (kGroups - 1);
  c.kc = lane_copy<DQK>(c.lane);
  c.vc = lane_copy<kDV>(c.lane);
  c.s_off = (c.lane & 31) * L::K::ROWB + c.half * 16;
  const int g = c.lane >> 4, j = c.lane & 15;
  c.v_off = ((g >> 1) * 4 + (j >> 2)) * L::V::ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;
  const int64_t w = (int64_t)pr.G - 1 - blockIdx.x;
  if (scorer) role<DQK, true>(c, pr, w, kbuf0, kbuf1, vbuf0, vbuf1, pbuf0, pbuf1);
  else role<DQK, false>(c, pr, w, kbuf0, kbuf1, vbuf0, vbuf1, pbuf0, pbuf1);
}

// out[b, i, h, :] = sum_s 2^(m_s - M) L_s / sum_s 2^(m_s - M) l_s over the
// partial states of row (b, h, i).  16 threads per row, 8 columns each.
template <bool OUT_F32>
__global__ __launch_bounds__(256)
void mha_merge_kernel(const float* __restrict__ part_L, const float* __restrict__ part_ml, int B, int H, int n_q,
                      int rb_per_bh, int T, int64_t U, int G, void* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= (int64_t)B * n_q * H) return;
  const int h = (int)(row % H);
  const int64_t bi = row / H;
  const int i = (int)(bi % n_q), b = (int)(bi / n_q);
  const int64_t rb = ((int64_t)b * H + h) * rb_per_bh + i / kRowsPerBlock;
  const int rl = i % kRowsPerBlock;
  const int64_t wa = unit_owner(rb * T, U, G), wb = unit_owner(rb * T + T - 1, U, G);
  float M = -INFINITY;
  for (int64_t w = wa; w <= wb; ++w) M = fmaxf(M, part_ml[(seg_slot(w, rb) * kRowsPerBlock + rl) * 2]);
  float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t w = wa; w <= wb; ++w) {
    const int64_t sl = seg_slot(w, rb);
    const float wt = exp2f(part_ml[(sl * kRowsPerBlock + rl) * 2] - M);
    l = fmaf(wt, part_ml[(sl * kRowsPerBlock + rl) * 2 + 1], l);
    const f32x4* src = reinterpret_cast<const f32x4*>(part_L + (sl * kRowsPerBlock + rl) * kDV + sub * 8);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(wt, x0[e], acc[e]);
      acc[4 + e] = fmaf(wt, x1[e], acc[4 + e]);
    }
  }
  const float inv = 1.f / l;
  const int64_t o = row * kDV + sub * 8;
  if (OUT_F32) {
    f32x4* dst = reinterpret_cast<f32x4*>((float*)out + o);
    dst[0] = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    dst[1] = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  } else {
    uint32_t wds[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wds[e] = bf16x2_bits(to_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv));
    *reinterpret_cast<uint4*>((u16*)out + o) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  }
}

// Queries in the attention kernel's layout: qt[(b*H + h)][i][e] =
// bf16(qfull[b, i, h, e]) with qfull = q (dense: an exact copy) or
// [q_h || RoPE3D(p_i) q_r,h] (non-absorbed latent); rows past n_q are zero.
// The softmax scale is applied to the fp32 scores, so no query is rounded
// after scaling.  Thread = 8 consecutive elements (16 bytes) of row i of
// sample blockIdx.y, for heads 4*blockIdx.z .. 4*blockIdx.z + 3 in turn (a
// rotated chunk's angles are evaluated once, in fp64, for those heads).
__global__ __launch_bounds__(256)
void mha_prep_q_kernel(const u16* __restrict__ q, const u16* __restrict__ q_r, const int* __restrict__ q_pos,
                       int H, int n_q, int dr, int rows_pad_h, RopeSpec rope, u16* __restrict__ qt) {
  constexpr int DH = 128, NQ = DH / 8;
  const int nch = NQ + dr / 8;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows_pad_h * nch) return;
  const int i = idx / nch, ch = idx - i * nch;
  const int b = blockIdx.y;
  const bool live = i < n_q, rot = ch >= NQ;
  const int er = (ch - NQ) * 8;
  float cs[4], sn[4];
  if (live && rot) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double ang = rope_angle((er >> 1) + k, q_pos[3 * i], q_pos[3 * i + 1], q_pos[3 * i + 2], rope);
      cs[k] = (float)cos(ang);
      sn[k] = (float)sin(ang);
    }
  }
  for (int h = blockIdx.z * 4; h < min(H, blockIdx.z * 4 + 4); ++h) {
    uint4 val = make_uint4(0, 0, 0, 0);
    if (live) {
      const int64_t tok = ((int64_t)b * n_q + i) * H + h;
      if (!rot) {
        val = *reinterpret_cast<const uint4*>(q + tok * DH + ch * 8);
      } else {
        const uint4 raw = *reinterpret_cast<const uint4*>(q_r + tok * dr + er);
        const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x2 two = __builtin_bit_cast(bf16x2, in[k]);
          const float a = (float)two[0], c = (float)two[1];
          o[k] = bf16x2_bits(to_bf16x2(fmaf(a, cs[k], -(c * sn[k])), fmaf(a, sn[k], c * cs[k])));
        }
        val = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    const int64_t bh = (int64_t)b * H + h;
    *reinterpret_cast<uint4*>(qt + (bh * rows_pad_h + i) * (nch * 8) + ch * 8) = val;
  }
}

// Per-head keys and values from the latent cache (non-absorbed form), head
// major so that the keys of one (batch, head) are contiguous:
//   K[b, h, j, 0:dh]   = W_UK[h] c_j,   K[b, h, j, dh:dh+dr] = k_R,j
//   V[b, h, j, :]      = W_UV[h] c_j
// Workgroup: 256 tokens (32 per wavefront) of one head, keys (blockIdx.z =
// 0) or values (1).  The head's 128 x d_c weight block is staged once in LDS
// (rows padded by 16 bytes so the 32 rows one b128 read touches spread over
// the banks); each wavefront keeps its tokens' latent rows in registers as
// the B operand and runs the four 32-output blocks through bf16 MFMA
// 32x32x16 with fp32 accumulation and one rounding to bf16.  Each block is
// staged in LDS so that four lanes store a token's 64 bytes of it together;
// the rows of consecutive tokens are adjacent.  The grid is about one round
// of workgroups: each loads its head's weights once and loops over 256-token
// blocks.  Key workgroups also copy k_R
// into their tokens' K rows.  K and V hold exactly n_k keys per sample.
template <int DC>
__global__ __launch_bounds__(512)
void mha_uplift_kernel(const u16* __restrict__ cache, int64_t cap, int n_k, int ntok, int H,
                       const u16* __restrict__ w_uk, const u16* __restrict__ w_uv,
                       u16* __restrict__ K, u16* __restrict__ V) {
  constexpr int W = DC + 32, DH = 128, DQK = DH + 32, KS = DC / 16, WROW = DC * 2 + 16, CPR = DC / 8;
  __shared__ __attribute__((aligned(16))) char wt[DH * WROW];
  constexpr int SROW = DQK * 2 + 16;   // staged output row: odd number of 16-byte slots
  __shared__ __attribute__((aligned(16))) char stage[8][32 * SROW];   // per wavefront: its 32 output rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int drow = is_v ? DH : DQK;    // elements per output row
  const u16* wsrc = (is_v ? w_uv : w_uk) + (int64_t)h * DH * DC;
  {
    // every piece of a thread is loaded before the first LDS store (one round
    // trip, not one per piece; the scheduler would otherwise pair them)
    constexpr int PER = DH * CPR / 512;
    static_assert(DH * CPR % 512 == 0, "whole pieces per thread");
    uint4 wv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = threadIdx.x + 512 * k, r = idx / CPR, ch = idx - r * CPR;
      wv[k] = *reinterpret_cast<const uint4*>(wsrc + r * DC + ch * 8);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = threadIdx.x + 512 * k, r = idx / CPR, ch = idx - r * CPR;
      *reinterpret_cast<uint4*>(wt + r * WROW + ch * 16) = wv[k];
    }
    __builtin_amdgcn_sched_group_barrier(0x020, PER, 0);
    __builtin_amdgcn_sched_group_barrier(0x200, PER, 0);
  }
  u16* out = is_v ? V : K;
  char* st = stage[wave];
  char* srow = st + (lane & 31) * SROW;
  const int pieces = drow / 8;         // 16-byte pieces per output row
  __syncthreads();
  // 256-token blocks blockIdx.x, blockIdx.x + gridDim.x, ...: the weight
  // stage is loaded once per workgroup, and the wavefronts run their blocks
  // without further barriers (each uses only its own staging area).
  // Latent row of this lane's token in block tb (tokens past the last re-read
  // it; their outputs are not stored).
  auto cache_row = [&](int tb) {
    const int my_tok = min(tb * 256 + wave * 32 + (lane & 31), ntok - 1);
    const int b = my_tok / n_k, j = my_tok - b * n_k;
    return cache + ((int64_t)b * cap + j) * W;
  };
  // The next block's latent rows load while this block computes.
  bf16x8 cf[KS];
  {
    const u16* crow = cache_row(blockIdx.x);
#pragma unroll
    for (int k = 0; k < KS; ++k) cf[k] = *reinterpret_cast<const bf16x8*>(crow + k * 16 + half * 8);
  }
#pragma unroll 1
  for (int tb = blockIdx.x; tb * 256 < ntok; tb += gridDim.x) {
    const int tok0 = tb * 256 + wave * 32;   // first token (b * n_k + j) of this wavefront
    const u16* crow = cache_row(tb);
    bf16x8 cn[KS];
    {
      const u16* nrow = cache_row(tb + gridDim.x);
#pragma unroll
      for (int k = 0; k < KS; ++k) cn[k] = *reinterpret_cast<const bf16x8*>(nrow + k * 16 + half * 8);
    }
    if (!is_v) {   // the positional key, shared by every head
      const uint4* kr = reinterpret_cast<const uint4*>(crow + DC + half * 16);
      uint4* kd = reinterpret_cast<uint4*>(srow + (DH + half * 16) * 2);
      kd[0] = kr[0];
      kd[1] = kr[1];
    }
#pragma unroll 1
    for (int ob = 0; ob < 4; ++ob) {
      const char* a = wt + (ob * 32 + (lane & 31)) * WROW + half * 16;
      f32x16 acc = {};
#pragma unroll
      for (int k = 0; k < KS; ++k) acc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(a + k * 32), cf[k], acc);
      // lane holds its token's outputs 32*ob + 8g + 4*half + t, t = 0..3
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(srow + (ob * 32 + g * 8 + half * 4) * 2) =
            make_uint2(bf16x2_bits(to_bf16x2(acc[4 * g], acc[4 * g + 1])),
                       bf16x2_bits(to_bf16x2(acc[4 * g + 2], acc[4 * g + 3])));
    }
    // the wavefront's LDS accesses run in order; these keep the compiler
    // from moving the copy-out reads above other lanes' writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int pc = lane; pc < 32 * pieces; pc += 64) {
      const int tw = pc / pieces, col = pc - tw * pieces;
      const int t = tok0 + tw;
      if (t < ntok) {
        const int ub = t / n_k, uj = t - ub * n_k;
        *reinterpret_cast<uint4*>(out + (((int64_t)ub * H + h) * n_k + uj) * drow + col * 8) =
            *reinterpret_cast<const uint4*>(st + tw * SROW + col * 16);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < KS; ++k) cf[k] = cn[k];
  }
}

}  // namespace mha

// ----------------------------------------------------------------- plans
MhaPlan make_mha_plan(int B, int H, int n_q, int n_k, int dqk, bool expanded) {
  MhaPlan p{};
  p.B = B; p.H = H; p.n_q = n_q; p.n_k = n_k; p.dqk = dqk;
  p.rb_per_bh = (n_q + kRowsPerBlock - 1) / kRowsPerBlock;
  p.rows_pad_h = p.rb_per_bh * kRowsPerBlock;
  p.nrb = (int64_t)B * H * p.rb_per_bh;
  p.T = (n_k + mha::kBN - 1) / mha::kBN;
  p.U = p.nrb * p.T;
  int64_t G = p.nrb;
  const int64_t rounds = (p.nrb + kPartitionCUs - 1) / kPartitionCUs;
  if ((double)p.nrb / (double)(rounds * kPartitionCUs) < 0.9) G = rounds * kPartitionCUs;
  if (G > p.U) G = p.U;
  if (G > p.nrb * kMaxSplitsPerBlock) G = p.nrb * kMaxSplitsPerBlock;
  p.G = (int32_t)G;
  const int64_t slots = G + p.nrb;
  p.off_qt = 0;
  p.off_L = align_up((int64_t)B * H * p.rows_pad_h * dqk * 2, 256);
  p.off_ml = align_up(p.off_L + slots * kRowsPerBlock * mha::kDV * 4, 256);
  p.off_k = align_up(p.off_ml + slots * kRowsPerBlock * 2 * 4, 256);
  p.off_v = p.off_k;
  p.total = p.off_k;
  if (expanded) {   // materialised per-head K [B, H, n_k, dqk] and V [B, H, n_k, 128] (head major)
    p.off_v = align_up(p.off_k + (int64_t)B * n_k * H * dqk * 2, 256);
    p.total = align_up(p.off_v + (int64_t)B * n_k * H * mha::kDV * 2, 256);
  }
  return p;
}

hipError_t launch_mha_prep_q(const MhaPlan& p, const MhaQueryArgs& a, hipStream_t s) {
  const int nch = p.dqk / 8;
  const dim3 grid((unsigned)((p.rows_pad_h * nch + 255) / 256), (unsigned)p.B, (unsigned)((p.H + 3) / 4));
  mha::mha_prep_q_kernel<<<grid, dim3(256), 0, s>>>((const u16*)a.q, (const u16*)a.q_r, a.q_pos, p.H, p.n_q,
                                                    p.dqk - 128, p.rows_pad_h, a.rope,
                                                    (u16*)((char*)a.workspace + p.off_qt));
  return hipGetLastError();
}

hipError_t launch_mha_uplift(const MhaPlan& p, const MhaUpliftArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const int ntok = p.B * p.n_k;
  // about one round of workgroups (two per compute unit), each looping over
  // 256-token blocks
  const int blocks = (ntok + 255) / 256;
  const int per_head = std::max(1, std::min(blocks, kPartitionCUs / (2 * p.H)));
  const dim3 grid((unsigned)per_head, p.H, 2), block(512);
  u16* K = (u16*)(ws + p.off_k);
  u16* V = (u16*)(ws + p.off_v);
  const u16* c = (const u16*)a.cache;
  const u16* wk = (const u16*)a.w_uk;
  const u16* wv = (const u16*)a.w_uv;
  switch (a.d_c) {
    case 64: mha::mha_uplift_kernel<64><<<grid, block, 0, s>>>(c, a.cap, p.n_k, ntok, p.H, wk, wv, K, V); break;
    case 128: mha::mha_uplift_kernel<128><<<grid, block, 0, s>>>(c, a.cap, p.n_k, ntok, p.H, wk, wv, K, V); break;
    case 192: mha::mha_uplift_kernel<192><<<grid, block, 0, s>>>(c, a.cap, p.n_k, ntok, p.H, wk, wv, K, V); break;
    case 256: mha::mha_uplift_kernel<256><<<grid, block, 0, s>>>(c, a.cap, p.n_k, ntok, p.H, wk, wv, K, V); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mha_attend(const MhaPlan& p, const MhaAttendArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  mha::Problem pr{};
  pr.q = (const u16*)(ws + p.off_qt);
  pr.k = (const u16*)a.k;
  pr.v = (const u16*)a.v;
  pr.cap = a.cap;
  pr.head_major = a.head_major;
  pr.H = p.H; pr.n_k = p.n_k; pr.rows_pad_h = p.rows_pad_h; pr.rb_per_bh = p.rb_per_bh; pr.T = p.T;
  pr.U = p.U; pr.G = p.G; pr.headroom = a.headroom; pr.qscale = a.qscale;
  pr.part_L = (float*)(ws + p.off_L);
  pr.part_ml = (float*)(ws + p.off_ml);
  switch (p.dqk) {
    case 128: mha::mha_attend_kernel<128><<<dim3(p.G), dim3(mha::kWaves * 64), 0, s>>>(pr); break;
    case 160: mha::mha_attend_kernel<160><<<dim3(p.G), dim3(mha::kWaves * 64), 0, s>>>(pr); break;
    default: return hipErrorInvalidValue;
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.B * p.n_q * p.H;
  const dim3 grid((unsigned)((rows + 15) / 16)), block(256);
  if (a.out_f32)
    mha::mha_merge_kernel<true><<<grid, block, 0, s>>>(pr.part_L, pr.part_ml, p.B, p.H, p.n_q, p.rb_per_bh, p.T, p.U,
                                                       p.G, a.out);
  else
    mha::mha_merge_kernel<false><<<grid, block, 0, s>>>(pr.part_L, pr.part_ml, p.B, p.H, p.n_q, p.rb_per_bh, p.T,
                                                        p.U, p.G, a.out);
  return hipGetLastError();
}

}  // namespace mla
