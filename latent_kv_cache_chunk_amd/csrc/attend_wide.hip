// Fused chunk attention for wide latents (d_c = 256): every wavefront owns
// 32 rows end to end.
//
// Same computation, partition and partial-state format as attend.hip (see
// there for the method's citations).  There, score and value wavefronts split
// the work of 64-row groups; at d_c = 256 a value wavefront's O accumulators
// alone would fill its 256 registers (64 rows x 256 columns of fp32), so this
// kernel keeps the single-role design instead: each wavefront computes the
// scores, the softmax and P.V for its own 32 rows.
//
// MFMA formulation (bf16 32x32x16, fp32 accumulate), per 32-row block:
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
// Staging: each tile of key_tile(256) keys is copied global -> LDS by
// direct-to-LDS 16-byte buffer loads (no registers), one row per key padded
// to an odd number of 16-byte slots so b128 reads of 16 consecutive rows hit
// distinct banks.  Two buffers: the next tile's loads are in flight while the
// current one is used; one barrier per tile.
//
// Softmax without in-loop rescaling: each row's reference max m is fixed by
// the first 32-key block of a segment and p = 2^(s - m) is accumulated as is
// (numerator and denominator share m, so the softmax is unchanged).  Later
// keys may score above m.  Every p >= 0, so a lane's running sum bounds each
// of its p: one check per segment -- a lane's sum above 2^headroom (32 by
// default) or an accumulator that is not finite -- decides whether the
// segment is redone exactly: a max-only sweep, then accumulation against the
// true max.  The same rule as the role-split kernels (attend.hip).
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {
namespace wide {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0), others free

template <int DC, int NW>
struct AttendTile {
  static constexpr int W = DC + 32;          // cached row width (elements)
  static constexpr int NCH = W / 8;          // 16-byte chunks per cached row
  static constexpr int NSLOT = NCH + 1;      // plus one pad slot: stride = 4 * odd dwords
  static constexpr int ROWB = NSLOT * 16;    // LDS bytes per key row
  static constexpr int BN = key_tile(DC);    // keys per tile
  static constexpr int NBLK = BN / 32;       // 32-key MFMA blocks per tile
  static constexpr int TILEB = BN * ROWB;    // LDS bytes per tile buffer
  static constexpr int ROWS_PER_LOAD = 64 / NSLOT;   // whole rows one 64-lane load copies
  static constexpr int NLOAD = (BN + ROWS_PER_LOAD - 1) / ROWS_PER_LOAD;
  static constexpr int LOADS_PER_WAVE = (NLOAD + NW - 1) / NW;
  static_assert(ROWS_PER_LOAD >= 1, "a cached row must fit one 64-lane load");
};

// Per-lane part of the direct-to-LDS copy: lane l copies chunk l % NSLOT of
// row l / NSLOT of the load's rows (the pad slot re-reads the row's last
// chunk); lanes past the last whole row stay idle (lane_row >= ROWS_PER_LOAD).
template <int DC, int NW>
__device__ inline int lane_copy_offset(int lane, int& lane_row) {
  using L = AttendTile<DC, NW>;
  lane_row = lane / L::NSLOT;
  const int ch = min(lane - lane_row * L::NSLOT, L::NCH - 1);
  return (lane_row * L::W + ch * 8) * 2;
}

// Enqueue the direct-to-LDS loads of key tile [key0, key0 + BN) into `tile`.
// Load i copies R = ROWS_PER_LOAD whole rows, [iR, iR + R), to LDS rows
// [iR, iR + R); in the last, partial tile rows past n_k re-read key n_k-1
// (their scores are masked).
template <int DC, int NW>
__device__ inline void issue_tile(__amdgpu_buffer_rsrc_t gsrc, int key0, int n_k, char* tile, int wave, int lane_off,
                                  int lane_row) {
  using L = AttendTile<DC, NW>;
  const bool partial = key0 + L::BN > n_k;
#pragma unroll
  for (int i = 0; i < L::LOADS_PER_WAVE; ++i) {
    const int ld = wave + NW * i;
    if (ld < L::NLOAD) {
      const int row0 = ld * L::ROWS_PER_LOAD;
      const uint32_t src = (uint32_t)(key0 + row0) * (uint32_t)(L::W * 2);
      int o = lane_off;
      if (partial) {
        const int key = key0 + row0 + lane_row;
        o += (min(key, n_k - 1) - key) * (L::W * 2);
      }
      if (lane_row < L::ROWS_PER_LOAD && row0 + lane_row < L::BN)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(gsrc, (lds_void*)(tile + row0 * L::ROWB), 16, src + (uint32_t)o, 0, 0, 0);
    }
  }
}

// Softmax state of one wavefront: QB 32-row MFMA blocks.
template <int DC, int QB>
struct WaveState {
  static constexpr int KS = (DC + 32) / 16, CB = DC / 32;
  bf16x8 qf[QB][KS];     // absorbed queries, MFMA B operands
  f32x16 oacc[QB][CB];   // O^T accumulators (latent columns x rows)
  float m_ref[QB];       // reference max (base 2), identical in lanes l and l^32
  float l_run[QB];       // this lane's part of the running sum
  int kv[QB];            // visible keys of the lane's row in each block (chunk-causal)
  int kv_min;            // smallest kv of the wavefront
  bool causal;
};

enum class Pass { kSingle, kMax, kAccum };

// Scores of one 32-key block for the wave's row blocks, the LDS operand loads
// PF k-steps ahead of the MFMA that uses them.  One accumulator chain per row
// block: a second, independent chain (summed at the end) spared consecutive
// MFMAs the wait on each other's results, but its 16 registers pushed two
// query fragments out to scratch, and their reloads (a vmcnt(0) wait, which
// also waits for the next tile's loads) sat in every block: 1.77 -> 1.68 ms
// at 480P without it.
template <int DC, int QB, int CHAINS = 1>
__device__ __forceinline__ void block_scores(const WaveState<DC, QB>& st, const char* kbase, f32x16 (&s)[QB]) {
  constexpr int KS = WaveState<DC, QB>::KS;
  constexpr int PF = 4;
  f32x16 acc[QB][CHAINS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[qb][c] = f32x16{};
  bf16x8 a[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) a[i] = *reinterpret_cast<const bf16x8*>(kbase + i * 32);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 cur = a[ks % PF];
    if (ks + PF < KS) a[ks % PF] = *reinterpret_cast<const bf16x8*>(kbase + (ks + PF) * 32);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc[qb][ks % CHAINS] = mfma_32x32x16(cur, st.qf[qb][ks], acc[qb][ks % CHAINS]);
  }
  // Issue order: PF loads, then (MFMA of step ks, load of step ks + PF).
#pragma unroll
  for (int i = 0; i < PF; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
    if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    s[qb] = acc[qb][0];
#pragma unroll
    for (int c = 1; c < CHAINS; ++c) s[qb] += acc[qb][c];
  }
}

// Softmax of one 32-key block: scores s (base-2 logits, masked keys = -inf)
// -> bf16 P operands.  kMax only raises the reference max.  kSingle fixes the
// reference max at the segment's first block.  It also flags a block max more
// than `headroom` above the reference: the running-sum bound at the segment's
// end implies that flag (such a p alone exceeds 2^headroom), and it is kept
// because the code generated without it spills the accumulators.
template <int DC, int QB, Pass P>
__device__ __forceinline__ void block_softmax(WaveState<DC, QB>& st, f32x16 (&s)[QB], bf16x8 (&pb)[QB][2],
                                              bool first_block, float headroom, bool& over) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (P != Pass::kAccum) {
      float mx = s[qb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[qb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (P == Pass::kMax) {
        st.m_ref[qb] = fmaxf(st.m_ref[qb], mx);
        continue;
      }
      st.m_ref[qb] = first_block ? mx : st.m_ref[qb];
      over |= mx > st.m_ref[qb] + headroom;
    }
    // a row with no visible key in this segment keeps m = -inf and p = 0
    const float m = st.m_ref[qb] == -INFINITY ? 0.f : st.m_ref[qb];
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
}

// O^T += V^T P^T for one 32-key block; V^T is read transposed from the tile.
template <int DC, int QB, int ROWB>
__device__ __forceinline__ void block_pv(WaveState<DC, QB>& st, const char* block_row0, int v_off,
                                         const bf16x8 (&pb)[QB][2]) {
  constexpr int CB = WaveState<DC, QB>::CB;
  // One stream of transposed reads over (part, column block), RA items ahead
  // of their MFMAs (the compiler otherwise waits on each read right after
  // issuing it).
  constexpr int NIT = 2 * CB, RA = 3;
  bf16x8 av[RA];
  auto vread = [&](int it) {
    const char* vb = block_row0 + (it / CB) * 16 * ROWB + v_off + (it % CB) * 64;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
#pragma unroll
  for (int it = 0; it < RA; ++it) av[it] = vread(it);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const bf16x8 a = av[it % RA];
    if (it + RA < NIT) av[it % RA] = vread(it + RA);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) st.oacc[qb][it % CB] = mfma_32x32x16(a, pb[qb][it / CB], st.oacc[qb][it % CB]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * RA, 0);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
    if (it + RA < NIT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// One staged tile, block by block (scores, softmax, P.V).  `left` = keys of
// the tile that exist; blocks past it are skipped, keys past it masked.
template <int DC, int QB, int NW, Pass P>
__device__ __forceinline__ void attend_tile(WaveState<DC, QB>& st, const char* tile, int key0, int left, int s_off,
                                            int v_off, int half, bool first_tile, float headroom, bool& over) {
  using L = AttendTile<DC, NW>;
  constexpr int ROWB = L::ROWB;
#pragma unroll 1
  for (int kb = 0; kb < L::NBLK; ++kb) {
    const int n_valid = min(32, left - kb * 32);
    if (n_valid <= 0) break;
    f32x16 s[QB];
    bf16x8 pb[QB][2];
    block_scores<DC, QB>(st, tile + kb * 32 * ROWB + s_off, s);
    const int bkey = key0 + kb * 32;
    if (st.causal && bkey + 32 > st.kv_min) {   // some row of the wavefront ends inside this block
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int thr = st.kv[qb] - bkey - half * 4;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if ((v >> 2) * 8 + (v & 3) >= thr) s[qb][v] = -INFINITY;
      }
    } else if (n_valid < 32) {
      const int thr = n_valid - half * 4;   // value v is key (v>>2)*8 + (v&3) + 4*half of the block
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if ((v >> 2) * 8 + (v & 3) >= thr) s[qb][v] = -INFINITY;
    }
    block_softmax<DC, QB, P>(st, s, pb, first_tile && kb == 0, headroom, over);
    if (P != Pass::kMax) block_pv<DC, QB, ROWB>(st, tile + kb * 32 * ROWB, v_off, pb);
  }
}

// Sweep tiles [t0, t1) of one segment through the two LDS buffers (each
// buffer a distinct LDS object, so that reads of one tile are not ordered
// behind the in-flight direct loads of the other).  kSingle returns true,
// identically in every wave, if some lane's running sum rose above
// 2^headroom or some accumulator is not finite.
template <int DC, int QB, int NW, Pass P>
__device__ __forceinline__ bool sweep(WaveState<DC, QB>& st, char* sbuf0, char* sbuf1, __amdgpu_buffer_rsrc_t gsrc, int t0,
                                      int t1, int n_k, int wave, int lane_off, int lane_row, int s_off, int v_off,
                                      int half, float headroom) {
  using L = AttendTile<DC, NW>;
  constexpr int BN = L::BN;
  bool over = false;
  issue_tile<DC, NW>(gsrc, t0 * BN, n_k, sbuf0, wave, lane_off, lane_row);
  wait_vmcnt0();
  __syncthreads();
#pragma unroll 1
  for (int t = t0; t < t1; t += 2) {
    // tile t is in sbuf0; tile t+1 goes to sbuf1
    if (t + 1 < t1) issue_tile<DC, NW>(gsrc, (t + 1) * BN, n_k, sbuf1, wave, lane_off, lane_row);
    attend_tile<DC, QB, NW, P>(st, sbuf0, t * BN, n_k - t * BN, s_off, v_off, half, t == t0, headroom, over);
    wait_vmcnt0();
    __syncthreads();
    if (t + 1 >= t1) break;
    if (t + 2 < t1) issue_tile<DC, NW>(gsrc, (t + 2) * BN, n_k, sbuf0, wave, lane_off, lane_row);
    attend_tile<DC, QB, NW, P>(st, sbuf1, (t + 1) * BN, n_k - (t + 1) * BN, s_off, v_off, half, false, headroom, over);
    wait_vmcnt0();
    __syncthreads();
  }
  if (P != Pass::kSingle) return false;
  // The segment's running sums (and accumulators, whose magnitudes are summed:
  // an inf or NaN among them carries through) against the bound.
  const float lim = __builtin_amdgcn_exp2f(headroom);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float asum = 0.f;
#pragma unroll
    for (int cb = 0; cb < WaveState<DC, QB>::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) asum += fabsf(st.oacc[qb][cb][v]);
    over |= !(st.l_run[qb] <= lim) || !(asum <= 3.0e38f);
  }
  return __syncthreads_or(over);
}

template <int DC, int QB>
__device__ __forceinline__ void reset_acc(WaveState<DC, QB>& st) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int cb = 0; cb < WaveState<DC, QB>::CB; ++cb) st.oacc[qb][cb] = f32x16{};
    st.l_run[qb] = 0.f;
  }
}

// QB = 32-row MFMA blocks per wavefront; QB = 1: 8 wavefronts of 32 rows,
// two per SIMD, so one wave's softmax overlaps the other's MFMAs.
template <int DC, int QB>
__global__ __launch_bounds__(512 / QB, 1)
void attend_wide_bf16_kernel(const u16* __restrict__ cache, int64_t cache_bstride, int n_k,
                        const u16* __restrict__ qt, int rows_pad_b, int rb_per_b,
                        float* __restrict__ part_L, float* __restrict__ part_ml,
                        int T, int64_t U, int G, float headroom, Visibility vis,
                        const int64_t* __restrict__ units, int64_t nrb, PartitionHeader* __restrict__ hdr) {
  constexpr int NW = 8 / QB;   // wavefronts per workgroup
  using L = AttendTile<DC, NW>;
  constexpr int W = L::W, KS = WaveState<DC, QB>::KS, CB = WaveState<DC, QB>::CB, ROWB = L::ROWB;
  static_assert(NW * QB * 32 == kRowsPerBlock, "a workgroup covers one row block");

  __shared__ __attribute__((aligned(1024))) char sbuf0[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char sbuf1[L::TILEB];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane_row;
  const int lane_off = lane_copy_offset<DC, NW>(lane, lane_row);
  // per-lane LDS offsets: b128 score operand, transposed latent operand
  const int s_off = (lane & 31) * ROWB + half * 16;
  const int g = lane >> 4, j = lane & 15;
  const int v_off = ((g >> 1) * 4 + (j >> 2)) * ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;

  // Workgroups are dispatched last unit range first: with chunk-causal
  // visibility the last row blocks see the most keys, and starting the
  // longest ranges first keeps the tail of the launch short.
  const int64_t w = (int64_t)G - 1 - blockIdx.x;
  const int64_t u = unit_begin(w, U, G);
  int64_t u_end = unit_begin(w + 1, U, G);
  WaveState<DC, QB> st;
  if (blockIdx.x == 0 && threadIdx.x == 0) *hdr = PartitionHeader{U, G, units != nullptr ? 1 : 0};

  int64_t rb = -1;
  while (u < u_end) {
    // this segment: the part of the range inside one row block (see Plan),
    // last row block first, so that ranges crossing a boundary start at key
    // tile 0 and the workgroups of an XCD sweep the cache nearly in step;
    // after the first, the row block before (row blocks are never empty)
    rb = rb < 0 ? rb_of_unit(units, T, nrb, u_end - 1) : rb - 1;
    const int64_t first = rb_first_unit(units, T, rb);
    const int64_t begin = max(u, first);
    int t0, t1;
    seg_tiles(units, first, begin, u_end, t0, t1);
    if (t1 <= t0) {   // start-up units only: no partial state
      u_end = begin;
      continue;
    }
    const int b = (int)(rb / rb_per_b);
    const int rbl = (int)(rb - (int64_t)b * rb_per_b);
    // Buffer resource over the sample's n_k rows (a byte count below 4 GiB,
    // checked by the host; the hardware reads it unsigned).  Tiles are copied
    // by buffer loads to LDS rather than global ones: after a global load to
    // LDS the compiler must assume the load may still touch LDS out of order,
    // so every wait on this wavefront's own LDS reads became a wait for all of
    // them (lgkmcnt(0)).  Traced attention at d_c = 256: -4.1%.
    const __amdgpu_buffer_rsrc_t gsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u16*>(cache + (int64_t)b * cache_bstride), 0, (int)((uint32_t)n_k * (uint32_t)(W * 2)),
        0x00020000);

    {
      const int64_t row0 = (int64_t)b * rows_pad_b + (int64_t)rbl * kRowsPerBlock + wave * 32 * QB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const u16* qrow = qt + (row0 + qb * 32 + (lane & 31)) * W + half * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) st.qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
      }
    }
    reset_acc<DC, QB>(st);
    // tiles past every row's visible keys are skipped (chunk-causal calls)
    const int te = min(t1, (vis.kv_max_of_block(rbl * kRowsPerBlock, n_k) + L::BN - 1) / L::BN);
    st.causal = vis.chunk_len != 0;
    int kvm = n_k;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      st.m_ref[qb] = -INFINITY;
      st.kv[qb] = vis.kv_of_row(rbl * kRowsPerBlock + wave * 32 * QB + qb * 32 + (lane & 31), n_k);
      kvm = min(kvm, st.kv[qb]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kvm = min(kvm, __shfl_xor(kvm, o));
    st.kv_min = kvm;
    if (te > t0 && sweep<DC, QB, NW, Pass::kSingle>(st, sbuf0, sbuf1, gsrc, t0, te, n_k, wave, lane_off, lane_row,
                                                    s_off, v_off, half, headroom)) {
      // A lane's running sum rose above 2^headroom (or an accumulator is not finite):
      // exact two-pass evaluation of this segment.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st.m_ref[qb] = -INFINITY;
      sweep<DC, QB, NW, Pass::kMax>(st, sbuf0, sbuf1, gsrc, t0, te, n_k, wave, lane_off, lane_row, s_off, v_off,
                                    half, headroom);
      reset_acc<DC, QB>(st);
      sweep<DC, QB, NW, Pass::kAccum>(st, sbuf0, sbuf1, gsrc, t0, te, n_k, wave, lane_off, lane_row, s_off,
                                      v_off, half, headroom);
    }

    // ---- write this segment's partial softmax state
    const int64_t slot = seg_slot(w, rb);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32);
      const int rl = wave * 32 * QB + qb * 32 + (lane & 31);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int c0 = cb * 32 + gg * 8 + half * 4;
          *reinterpret_cast<f32x4*>(part_L + part_L_index(slot, rl, c0, DC)) =
              f32x4{st.oacc[qb][cb][4 * gg], st.oacc[qb][cb][4 * gg + 1], st.oacc[qb][cb][4 * gg + 2],
                    st.oacc[qb][cb][4 * gg + 3]};
        }
      if (half == 0) {
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 0] = st.m_ref[qb];
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 1] = l_tot;
      }
    }
    u_end = begin;
  }
}

}  // namespace wide

hipError_t launch_attend_wide_bf16(const Plan& p, const AttendArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const u16* cache = (const u16*)a.cache;
  const u16* qt = (const u16*)(ws + p.off_qt);
  float* L = (float*)(ws + p.off_L);
  float* ml = (float*)(ws + p.off_ml);
  const int64_t* units = p.causal ? (const int64_t*)(ws + p.off_units) : nullptr;
  PartitionHeader* hdr = (PartitionHeader*)(ws + p.off_hdr);
  if (p.d_c != 256) return hipErrorInvalidValue;
  wide::attend_wide_bf16_kernel<256, 1><<<dim3(p.G), dim3(512), 0, s>>>(cache, a.cache_bstride, p.n_k, qt,
                                                                        p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U,
                                                                        p.G, a.headroom, a.vis, units, p.nrb, hdr);
  return hipGetLastError();
}

}  // namespace mla
