// Fused chunk attention over the latent cache.
//
// For every row r = (batch, head, query) of the current chunk and every
// visible key j (all cached chunks plus the chunk itself -- chunk-causal,
// bidirectional inside the chunk; VideoMLA atlas.scime.ai summary, first
// paragraph) the score is the dot product of the absorbed query q~_r with the
// cached row [c_j || k_R,j]; the kernel keeps a base-2 softmax and
// accumulates L_r = sum_j p_rj c_j in fp32.  Every head reads the same latent
// rows (VideoMLA arXiv abstract: one latent and one positional key shared by
// all heads), so a workgroup packs 256 rows of any heads and streams each key
// tile through LDS once for all of them.
//
// Wavefront roles.  The 256 rows form four groups of 64.  Each group has a
// score wavefront and a value wavefront, placed on the same SIMD:
//   score:  S^T[key][row] = K_blk[key][:] . q~[row][:]  (bf16 MFMA 32x32x16,
//           A = key rows read from LDS, B = q~ rows held in registers), then
//           p = 2^(s - m) in fp32, the row sums, and P in bf16 written to LDS;
//   value:  O^T[c][row] += V^T[c][key] . P^T[key][row]  (A = latent columns
//           read transposed from the same LDS tile with ds_read_tr16_b64,
//           B = P read back from LDS).
// The score wavefront never holds O and the value wavefront never holds q~,
// so each fits its registers with room to spare, and while one wavefront of
// a SIMD is in its softmax the other keeps the matrix core busy.  Each LDS
// operand read feeds two MFMAs (the group's two 32-row halves).  At d_c <= 128
// the scores are cheap against the softmax, so each half gets a score
// wavefront of its own (three wavefronts per SIMD): the exponentials of a
// group then run in two wavefronts beside the value wavefront's MFMAs.
//
// With keys on the MFMA rows one lane holds 16 keys of one row, so row sums
// are lane-local.  Lane-half h of the S^T accumulator holds keys
// {8g + 4h + t}; the transposed loads fetch exactly those keys for the P.V
// k-step, so each lane's P values go to LDS and come back to the same lane
// of the value wavefront unchanged.
//
// Pipeline.  Key tiles are copied global -> LDS by direct-to-LDS 16-byte
// loads (no registers; buffer loads at d_c >= 128, global ones at d_c = 64,
// whichever measured faster), one row per key padded to an odd number of
// 16-byte slots so b128 reads of 16 consecutive rows hit distinct banks.  In
// step k the score wavefronts work on tile k, the value wavefronts on tile
// k-1 (with the P of step k-1), and tile k+1 is in flight (its loads issued
// by the value wavefronts): three key buffers, two P buffers, one barrier per
// step.
//
// Softmax without rescaling.  The accumulators are never rescaled.  Each
// row's reference max m is fixed by the first 32-key block of a segment and
// p = 2^(s - m) is accumulated as is: numerator and denominator share m, so
// the softmax is unchanged.  After that first block the score MFMAs start
// from -m instead of 0 and deliver s - m themselves (one subtraction per
// score less on the score wavefront).  Later keys may score above m; this is
// safe while p stays far inside the fp32 range.  Since every p >= 0, a lane's
// running sum bounds each of its p, so one check per segment suffices: if a
// lane's sum exceeds 2^headroom (32 by default) or an accumulator is not
// finite, the segment is redone exactly -- a max-only sweep, then
// accumulation against the true max.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0), others free

constexpr int kGroups = 4;         // row groups (score + value wavefronts each)
constexpr int kGroupRows = 64;     // rows per group: two 32-row MFMA blocks
// 32-row halves per score wavefront: at d_c <= 128 each group has two score
// wavefronts, one per half, so the softmax of a group runs in two wavefronts
// beside the value wavefront (three per SIMD; the value accumulators of 64
// rows x d_c columns still fit the third of the register file each gets, with
// the spills of d_c = 128 confined to segment set-up and epilogue code).
template <int DC> constexpr int score_halves() { return DC <= 128 ? 1 : 2; }
template <int DC> constexpr int attend_waves() { return kGroups * (score_halves<DC>() == 1 ? 3 : 2); }
static_assert(kGroups * kGroupRows == kRowsPerBlock, "a workgroup covers one row block");

template <int DC>
struct AttendTile {
  static constexpr int W = DC + 32;          // cached row width (elements)
  static constexpr int NCH = W / 8;          // 16-byte chunks per cached row
  static constexpr int NSLOT = NCH + 1;      // plus one pad slot: stride = 4 * odd dwords
  static constexpr int ROWB = NSLOT * 16;    // LDS bytes per key row
  static constexpr int BN = key_tile(DC);    // keys per tile
  static constexpr int NBLK = BN / 32;       // 32-key MFMA blocks per tile
  static constexpr int TILEB = BN * ROWB;    // LDS bytes per key buffer
  static constexpr int ROWS_PER_LOAD = 64 / NSLOT;   // whole rows one 64-lane load copies
  static constexpr int NLOAD = (BN + ROWS_PER_LOAD - 1) / ROWS_PER_LOAD;
  static constexpr int LOADS_PER_WAVE = (NLOAD + kGroups - 1) / kGroups;   // value wavefronts issue the loads
  static constexpr int KS = W / 16;          // score k-steps
  static constexpr int CB = DC / 32;         // 32-column latent blocks of O^T
  static constexpr int PBLK = kGroups * 2 * 2 * 64 * 16;   // P bytes of one block: groups x halves x k-steps x lanes
  static constexpr int PBUF = NBLK * PBLK;                 // LDS bytes per P buffer
  static_assert(ROWS_PER_LOAD >= 1, "a cached row must fit one 64-lane load");
  static_assert(3 * TILEB + 2 * PBUF <= 160 * 1024, "buffers exceed LDS");
};

// Per-lane part of the direct-to-LDS copy: lane l copies chunk l % NSLOT of
// row l / NSLOT of the load's rows (the pad slot re-reads the row's last
// chunk); lanes past the last whole row stay idle (lane_row >= ROWS_PER_LOAD).
// Returns the chunk's byte offset inside its row.
template <int DC>
__device__ inline int lane_copy_chunk(int lane, int& lane_row) {
  using L = AttendTile<DC>;
  lane_row = lane / L::NSLOT;
  return min(lane - lane_row * L::NSLOT, L::NCH - 1) * 16;
}

// Wave-invariant addressing of one sweep.
struct SweepCtx {
  const char* gbase;             // cache rows of this sample
  __amdgpu_buffer_rsrc_t gsrc;   // buffer resource over the visible cache rows of this sample
  int n_k;
  bool causal;         // keys limited per row (chunk-causal visibility)
  int kv[2];           // score lanes: visible keys of the lane's row in each of the wavefront's halves
  int qb0;             // score wavefronts: first 32-row half of the group they cover
  int kv_min;          // score wavefronts: smallest kv of the wavefront
  int wave, lane, half, group;
  int lane_chunk, lane_row;
  int s_off;           // b128 score operand offset inside a block
  int v_off;           // transposed latent operand offset inside a block
};

// Buffer resource over rows [0, n_k) of sample b.  At d_c >= 128 the tiles
// are copied by buffer loads to LDS rather than global ones: after a global
// load to LDS the compiler must assume the load may still touch LDS out of
// order, so every wait on this wavefront's own LDS reads became a wait for
// all of them (lgkmcnt(0)) until the next wait for vector memory.  Traced
// attention with buffer loads: 480P -0.4%, d_c = 128 -0.4%, block-causal
// -2.3%, but d_c = 64 +1.2%, which keeps global loads.
template <int DC> constexpr bool buffer_tile_loads() { return DC >= 128; }
template <int DC>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sample_rows(const u16* cache, int64_t cache_bstride, int b,
                                                              int n_k) {
  // byte count below 4 GiB (checked by the host), the hardware reads it unsigned
  const uint32_t bytes = (uint32_t)n_k * (uint32_t)(AttendTile<DC>::W * 2);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(cache + (int64_t)b * cache_bstride), 0, (int)bytes,
                                           0x00020000);
}

// Enqueue this value wavefront's share of the direct-to-LDS loads of key tile
// t into `tile`.  Only the value wavefronts issue loads: the score wavefront
// is each step's critical path (its scores, softmax and P stores take longer
// than the value product), and the loads' issue costs it about 300 cycles a
// step.  Load i copies R = ROWS_PER_LOAD whole rows, [iR, iR + R), to
// LDS rows [iR, iR + R); in the last, partial tile rows past n_k re-read key
// n_k-1 (their scores are masked).  Source addresses are the sample's base
// plus a 32-bit unsigned offset (a sample's cache is below 4 GiB), inside the
// buffer resource's n_k rows.
template <int DC>
__device__ inline void issue_tile(const SweepCtx& c, int t, char* tile) {
  using L = AttendTile<DC>;
  const int key0 = t * L::BN;
#pragma unroll
  for (int i = 0; i < L::LOADS_PER_WAVE; ++i) {
    const int ld = c.group + kGroups * i;
    if (ld < L::NLOAD) {
      const int row0 = ld * L::ROWS_PER_LOAD;
      const uint32_t key = (uint32_t)min(key0 + row0 + c.lane_row, c.n_k - 1);
      const uint32_t off = key * (uint32_t)(L::W * 2) + (uint32_t)c.lane_chunk;
      if (c.lane_row < L::ROWS_PER_LOAD && row0 + c.lane_row < L::BN) {
        if constexpr (buffer_tile_loads<DC>())
          __builtin_amdgcn_raw_ptr_buffer_load_lds(c.gsrc, (lds_void*)(tile + row0 * L::ROWB), 16, off, 0, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(c.gbase + off, (lds_void*)(tile + row0 * L::ROWB), 16, 0, 0);
      }
    }
  }
}

enum class Pass { kSingle, kMax, kAccum };

// Byte offset of lane `lane`'s 16-byte P operand (row half qb, k-step part)
// of group g inside one block of a P buffer.
__device__ __forceinline__ int p_slot(int g, int qb, int part, int lane) {
  return (((g * 2 + qb) * 2 + part) * 64 + lane) * 16;
}

// Keys of the block at or past n_valid get score -inf (p = 0).  Value v of
// lane-half h is key (v>>2)*8 + 4h + (v&3) of the block.
__device__ __forceinline__ void mask_block(f32x16& s, int n_valid, int half) {
  const int thr = n_valid - half * 4;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if ((v >> 2) * 8 + (v & 3) >= thr) s[v] = -INFINITY;
}

// Row max of a block (both lane halves).
__device__ __forceinline__ float block_max(const f32x16& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float b = fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]));
  const float c = fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11]));
  const float d = fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]));
  const float m = fmaxf(fmaxf(a, b), fmaxf(c, d));
  return fmaxf(m, __shfl_xor(m, 32));
}

// ---------------------------------------------------------------- score role
template <int DC>
struct ScoreState {
  static constexpr int NQB = score_halves<DC>();
  bf16x8 qf[NQB][AttendTile<DC>::KS];   // absorbed queries of the wavefront's halves (MFMA B operands)
  float m_ref[NQB];                     // reference max (base 2), identical in lanes l and l^32
  float l_run[NQB];                     // this lane's part of the running sum
  f32x16 neg_m[NQB];                    // -m in every element: the accumulator a block's products start from
};

// Accumulator start -m for every later block of a segment (m = 0 for a row
// with no visible key, whose scores are all -inf).
template <int DC>
__device__ __forceinline__ void set_neg_m(ScoreState<DC>& st, int qb) {
  const float m = st.m_ref[qb] == -INFINITY ? 0.f : st.m_ref[qb];
#pragma unroll
  for (int v = 0; v < 16; ++v) st.neg_m[qb][v] = -m;
}

// Score operand loads in flight ahead of their MFMAs.  Six at d_c = 64 and
// 192 (against four: 480P attention -0.6%, d_c = 64 -1.2%); four at d_c = 128,
// where six was 0.5% slower.
template <int DC> constexpr int score_prefetch() { return DC == 128 ? 4 : 6; }

// Scores, softmax and P of every block of tile t (LDS `tile`), P to `pbuf`.
// MASK: some key of the tile is past n_k or past a row's visible keys.  The
// unmasked form has no masking branch after its products, so the scores
// stay in the registers the products wrote (a branch that may rewrite them
// made the compiler copy all 32 after every tile's second block).
// FIRST: the segment's first tile in a single-pass sweep; its first block
// sets the reference max.  Every other block of a pass that accumulates
// starts its products from -m, so the MFMAs deliver s - m and the softmax
// takes 2^x of the accumulator directly.
template <int DC, Pass P, bool MASK, bool FIRST>
__device__ __forceinline__ void score_tile(ScoreState<DC>& st, const char* tile, char* pbuf, int t,
                                           const SweepCtx& c) {
  using L = AttendTile<DC>;
  constexpr int KS = L::KS, PF = score_prefetch<DC>(), NQB = ScoreState<DC>::NQB;
  const int left = c.n_k - t * L::BN;
  // One stream of K operand reads over the tile's blocks: read g (block g /
  // KS, k-step g % KS) goes to slot g % PF and is issued PF k-steps ahead of
  // its MFMAs, so the next block's first reads are in flight during this
  // block's softmax (left to itself the compiler keeps two reads in flight;
  // the stream was 3.5% faster).  Reads of a block past the tile's last key
  // are issued and unused.
  bf16x8 a[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) a[i] = *reinterpret_cast<const bf16x8*>(tile + c.s_off + i * 32);
#pragma unroll
  for (int kb = 0; kb < L::NBLK; ++kb) {
    if (MASK && kb > 0 && kb * 32 >= left) break;
    // fresh: the products start from 0 (the max pass, and the block that sets m)
    const bool fresh = P == Pass::kMax || (FIRST && kb == 0);
    f32x16 s[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) s[qb] = fresh ? f32x16{} : st.neg_m[qb];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int g = kb * KS + ks;
      const bf16x8 cur = a[g % PF];
      const int gn = g + PF;
      if (gn < L::NBLK * KS)
        a[g % PF] = *reinterpret_cast<const bf16x8*>(tile + (gn / KS) * 32 * L::ROWB + c.s_off + (gn % KS) * 32);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[qb] = mfma_32x32x16(cur, st.qf[qb][ks], s[qb]);
    }
    if (kb == 0) __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, NQB, 0);
      if (kb * KS + ks + PF < L::NBLK * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    const int key0 = t * L::BN + kb * 32;
    if constexpr (MASK) {
      if (c.causal) {
        if (key0 + 32 > c.kv_min) {   // some row of the wavefront ends inside this block
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) mask_block(s[qb], c.kv[qb] - key0, c.half);
        }
      } else if (left - kb * 32 < 32) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) mask_block(s[qb], left - kb * 32, c.half);
      }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (P == Pass::kMax) {
        st.m_ref[qb] = fmaxf(st.m_ref[qb], block_max(s[qb]));
        continue;
      }
      float p[16];
      if (fresh) {
        // a row with no visible key in this segment keeps m = -inf and p = 0
        st.m_ref[qb] = block_max(s[qb]);
        set_neg_m(st, qb);
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(s[qb][v] + st.neg_m[qb][v]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(s[qb][v]);
      }
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
        *reinterpret_cast<bf16x8*>(pbuf + kb * L::PBLK + p_slot(c.group, (NQB == 1 ? c.qb0 : 0) + qb, part, c.lane)) = pv;
      }
    }
  }
}

// ---------------------------------------------------------------- value role
template <int DC>
struct ValueState {
  f32x16 oacc[2][AttendTile<DC>::CB];   // O^T accumulators of the group's two halves
};

// P.V of every block of tile t (LDS `tile`), P from `pbuf`.
template <int DC>
__device__ __forceinline__ void value_tile(ValueState<DC>& st, const char* tile, const char* pbuf, int t,
                                           const SweepCtx& c) {
  using L = AttendTile<DC>;
  const int left = c.n_k - t * L::BN;
#pragma unroll
  for (int kb = 0; kb < L::NBLK; ++kb) {
    if (kb > 0 && kb * 32 >= left) break;
    const char* pb = pbuf + kb * L::PBLK;
    const char* blk = tile + kb * 32 * L::ROWB + c.v_off;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const bf16x8 p0 = *reinterpret_cast<const bf16x8*>(pb + p_slot(c.group, 0, part, c.lane));
      const bf16x8 p1 = *reinterpret_cast<const bf16x8*>(pb + p_slot(c.group, 1, part, c.lane));
      const char* vbase = blk + part * 16 * L::ROWB;
      bf16x8 av[L::CB];
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + cb * 64));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + 8 * L::ROWB + cb * 64));
        av[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) {
        st.oacc[0][cb] = mfma_32x32x16(av[cb], p0, st.oacc[0][cb]);
        st.oacc[1][cb] = mfma_32x32x16(av[cb], p1, st.oacc[1][cb]);
      }
      // Issue order: the P reads and the transposed reads of three column
      // blocks, then two MFMAs and the reads three column blocks ahead, so
      // that each pair of MFMAs waits on reads issued two pairs earlier (the
      // compiler otherwise waits on every read right after issuing it).
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (cb + 3 < L::CB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  }
}

// ------------------------------------------------------------------ sweeps
// One step of a segment's sweep: (value wavefronts) start tile k+1 into `nxt`, do this role's
// work (score: tile k in `cur`, P to P[k % 2]; value: tile k-1 in `prv`, P
// from P[(k-1) % 2]), then wait for the loads and barrier.  Steps run
// k = 0 .. n (n tiles); returns true after step n.
template <int DC, Pass P, bool SCORE, bool FIRST, class State>
__device__ __forceinline__ bool sweep_step(State& st, int k, int n, int t0, char* cur, char* nxt, char* prv,
                                           char* pbuf, const SweepCtx& c) {
  if (!SCORE && k + 1 < n) issue_tile<DC>(c, t0 + k + 1, nxt);
  if constexpr (SCORE) {
    if (k < n) {
      constexpr int BN = AttendTile<DC>::BN;
      const int t = t0 + k;
      char* pb = pbuf + ((k & 1) ? AttendTile<DC>::PBUF : 0);
      constexpr bool F = FIRST && P == Pass::kSingle;
      if (c.causal ? t * BN + BN > c.kv_min : c.n_k - t * BN < BN)
        score_tile<DC, P, true, F>(st, cur, pb, t, c);
      else
        score_tile<DC, P, false, F>(st, cur, pb, t, c);
    }
  } else {
    if (P != Pass::kMax && k >= 1) value_tile<DC>(st, prv, pbuf + ((k & 1) ? 0 : AttendTile<DC>::PBUF), t0 + k - 1, c);
  }
  wait_vmcnt0();
  __syncthreads();
  return k >= n;
}

// Tiles [t0, t1) of one segment.  The three key buffers are distinct LDS
// objects and each step names them statically (the loop is unrolled by
// three), so reads of one are not ordered behind the in-flight direct loads
// of another.  Score and value wavefronts run the same steps and barriers.
// Step 0 (the segment's first tile) is peeled off the loop.
template <int DC, Pass P, bool SCORE, class State>
__device__ __forceinline__ void sweep(State& st, char* k0, char* k1, char* k2, char* pbuf, int t0, int t1,
                                      const SweepCtx& c) {
  const int n = t1 - t0;
  if (!SCORE) issue_tile<DC>(c, t0, k0);
  wait_vmcnt0();
  __syncthreads();
  if (sweep_step<DC, P, SCORE, true>(st, 0, n, t0, k0, k1, k2, pbuf, c)) return;
#pragma unroll 1
  for (int k = 1;; k += 3) {
    if (sweep_step<DC, P, SCORE, false>(st, k, n, t0, k1, k2, k0, pbuf, c)) break;
    if (sweep_step<DC, P, SCORE, false>(st, k + 1, n, t0, k2, k0, k1, pbuf, c)) break;
    if (sweep_step<DC, P, SCORE, false>(st, k + 2, n, t0, k0, k1, k2, pbuf, c)) break;
  }
}

// Segments of workgroup w: its contiguous unit range, cut at row-block
// boundaries (see Plan), visited last row block first.  A range that crosses
// a boundary then starts at key tile 0, and its earlier row block's tail
// follows at a fixed tile offset (the unit count per workgroup is nearly the
// same for all), so the workgroups of one XCD sweep the cache nearly in step
// and share its tiles in their L2 instead of each streaming the whole cache.
struct SegmentIter {
  int64_t u, u_end;
  int T, rb_per_b;
  const int64_t* units;   // first unit of each row block (chunk-causal), or nullptr
  int64_t nrb;
  int64_t rb;
  int t0, t1, b, rbl;
  // Next segment that holds a key tile (one of start-up units only is skipped).
  // After the first, each segment lies in the row block before the last one:
  // row blocks are contiguous and never empty.
  __device__ bool next() {
    while (u < u_end) {
      rb = rb < 0 ? rb_of_unit(units, T, nrb, u_end - 1) : rb - 1;
      const int64_t first = rb_first_unit(units, T, rb);
      const int64_t begin = max(u, first);
      seg_tiles(units, first, begin, u_end, t0, t1);
      u_end = begin;
      if (t1 > t0) {
        b = (int)(rb / rb_per_b);
        rbl = (int)(rb - (int64_t)b * rb_per_b);
        return true;
      }
    }
    return false;
  }
};

// End of the segment's tiles that some row of the row block can see (t1 when
// every key is visible); a segment that ends at or before t0 is empty.
template <int DC>
__device__ __forceinline__ int visible_end(const SegmentIter& it, const Visibility& vis, int n_k) {
  constexpr int BN = AttendTile<DC>::BN;
  const int kv = vis.kv_max_of_block(it.rbl * kRowsPerBlock, n_k);
  return min(it.t1, (kv + BN - 1) / BN);
}

// OR of `v` over the workgroup with one barrier: each wavefront posts its own
// vote in one of two LDS vote sets (alternating per call, so a set is
// rewritten only after every wavefront has passed the next call's barrier,
// i.e. has read it), then every thread reads all votes.
template <int NW>
__device__ __forceinline__ bool workgroup_any(bool v, int* votes, int& parity) {
  const int wave = threadIdx.x >> 6;
  const int any = __any(v) ? 1 : 0;
  int* set = votes + parity * NW;
  if ((threadIdx.x & 63) == 0) set[wave] = any;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r |= set[w];
  parity ^= 1;
  return r != 0;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

template <int DC>
__device__ __forceinline__ void score_role(SweepCtx& c, SegmentIter it, const u16* __restrict__ cache,
                                           int64_t cache_bstride, const u16* __restrict__ qt, int rows_pad_b,
                                           float* __restrict__ part_ml, int64_t w, float headroom,
                                           const Visibility& vis, char* k0, char* k1, char* k2, char* pbuf,
                                           int* votes) {
  using L = AttendTile<DC>;
  constexpr int NQB = ScoreState<DC>::NQB;
  ScoreState<DC> st;
  int parity = 0;
  while (it.next()) {
    c.gbase = reinterpret_cast<const char*>(cache + (int64_t)it.b * cache_bstride);
    c.gsrc = sample_rows<DC>(cache, cache_bstride, it.b, c.n_k);
    const int te = visible_end<DC>(it, vis, c.n_k);
    const int64_t row0 = (int64_t)it.b * rows_pad_b + (int64_t)it.rbl * kRowsPerBlock + c.group * kGroupRows;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int half_row = ((NQB == 1 ? c.qb0 : 0) + qb) * 32 + (c.lane & 31);
      const u16* qrow = qt + (row0 + half_row) * L::W + c.half * 8;
#pragma unroll
      for (int ks = 0; ks < L::KS; ++ks) st.qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
      st.l_run[qb] = 0.f;
      st.m_ref[qb] = -INFINITY;
      c.kv[qb] = vis.kv_of_row(it.rbl * kRowsPerBlock + c.group * kGroupRows + half_row, c.n_k);
    }
    c.kv_min = wave_min(NQB == 2 ? min(c.kv[0], c.kv[1]) : c.kv[0]);
    if (te > it.t0) sweep<DC, Pass::kSingle, true>(st, k0, k1, k2, pbuf, it.t0, te, c);
    const float lim = __builtin_amdgcn_exp2f(headroom);
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) over |= !(st.l_run[qb] <= lim);
    if (workgroup_any<attend_waves<DC>()>(over, votes, parity)) {
      // A running sum rose past 2^headroom: exact two-pass evaluation.
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) st.m_ref[qb] = -INFINITY;
      sweep<DC, Pass::kMax, true>(st, k0, k1, k2, pbuf, it.t0, te, c);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        st.l_run[qb] = 0.f;
        set_neg_m(st, qb);
      }
      sweep<DC, Pass::kAccum, true>(st, k0, k1, k2, pbuf, it.t0, te, c);
    }
    const int64_t slot = seg_slot(w, it.rb);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float l_tot = st.l_run[qb] + __shfl_xor(st.l_run[qb], 32);
      const int rl = c.group * kGroupRows + ((NQB == 1 ? c.qb0 : 0) + qb) * 32 + (c.lane & 31);
      if (c.half == 0) {
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 0] = st.m_ref[qb];
        part_ml[(slot * kRowsPerBlock + rl) * 2 + 1] = l_tot;
      }
    }
  }
}

template <int DC>
__device__ __forceinline__ void value_role(SweepCtx& c, SegmentIter it, const u16* __restrict__ cache,
                                           int64_t cache_bstride, float* __restrict__ part_L, int64_t w,
                                           const Visibility& vis, char* k0, char* k1, char* k2, char* pbuf,
                                           int* votes) {
  using L = AttendTile<DC>;
  ValueState<DC> st;
  int parity = 0;
  while (it.next()) {
    c.gbase = reinterpret_cast<const char*>(cache + (int64_t)it.b * cache_bstride);
    c.gsrc = sample_rows<DC>(cache, cache_bstride, it.b, c.n_k);
    const int te = visible_end<DC>(it, vis, c.n_k);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb) st.oacc[qb][cb] = f32x16{};
    if (te > it.t0) sweep<DC, Pass::kSingle, false>(st, k0, k1, k2, pbuf, it.t0, te, c);
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) bad |= !(fabsf(st.oacc[qb][cb][v]) <= 3.0e38f);
    if (workgroup_any<attend_waves<DC>()>(bad, votes, parity)) {
      sweep<DC, Pass::kMax, false>(st, k0, k1, k2, pbuf, it.t0, te, c);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int cb = 0; cb < L::CB; ++cb) st.oacc[qb][cb] = f32x16{};
      sweep<DC, Pass::kAccum, false>(st, k0, k1, k2, pbuf, it.t0, te, c);
    }
    const int64_t slot = seg_slot(w, it.rb);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int rl = c.group * kGroupRows + qb * 32 + (c.lane & 31);
#pragma unroll
      for (int cb = 0; cb < L::CB; ++cb)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int c0 = cb * 32 + gg * 8 + c.half * 4;
          *reinterpret_cast<f32x4*>(part_L + part_L_index(slot, rl, c0, DC)) =
              f32x4{st.oacc[qb][cb][4 * gg], st.oacc[qb][cb][4 * gg + 1], st.oacc[qb][cb][4 * gg + 2],
                    st.oacc[qb][cb][4 * gg + 3]};
        }
    }
  }
}

// One workgroup = 256 rows x a contiguous range of (row-block, key-tile)
// units; each row-block segment leaves a partial softmax state (m, l, L) in
// its slot: score wavefronts write (m, l), value wavefronts write L.
template <int DC>
__global__ __launch_bounds__(attend_waves<DC>() * 64, 1)
void attend_bf16_kernel(const u16* __restrict__ cache, int64_t cache_bstride, int n_k,
                        const u16* __restrict__ qt, int rows_pad_b, int rb_per_b,
                        float* __restrict__ part_L, float* __restrict__ part_ml,
                        int T, int64_t U, int G, float headroom, Visibility vis,
                        const int64_t* __restrict__ units, int64_t nrb, PartitionHeader* __restrict__ hdr) {
  using L = AttendTile<DC>;
  __shared__ __attribute__((aligned(1024))) char kbuf0[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[L::TILEB];
  __shared__ __attribute__((aligned(1024))) char kbuf2[L::TILEB];
  // The two P buffers are one LDS object addressed by offset: a P read through
  // a pointer chosen between two objects would not be known to miss the key
  // buffers, and the compiler would wait for the in-flight tile loads first.
  __shared__ __attribute__((aligned(1024))) char pbuf[2 * L::PBUF];
  __shared__ int votes[2 * attend_waves<DC>()];   // per-segment fallback vote (two alternating sets)

  SweepCtx c;
  c.n_k = n_k;
  c.causal = vis.chunk_len != 0;
  c.kv[0] = c.kv[1] = c.kv_min = n_k;
  c.lane = threadIdx.x & 63;
  c.half = c.lane >> 5;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wavefront w runs on SIMD w % 4: group g's wavefronts are g, g + 4 (and g + 8)
  constexpr int kScoreWaves = kGroups * (3 - score_halves<DC>());
  const bool scorer = c.wave < kScoreWaves;
  c.group = c.wave & (kGroups - 1);
  c.qb0 = score_halves<DC>() == 1 ? (c.wave >> 2) & 1 : 0;
  c.lane_chunk = lane_copy_chunk<DC>(c.lane, c.lane_row);
  c.s_off = (c.lane & 31) * L::ROWB + c.half * 16;
  const int g = c.lane >> 4, j = c.lane & 15;
  c.v_off = ((g >> 1) * 4 + (j >> 2)) * L::ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;

  // Workgroups are dispatched last unit range first: with chunk-causal
  // visibility the last row blocks see the most keys, and starting the
  // longest ranges first keeps the tail of the launch short.
  const int64_t w = (int64_t)G - 1 - blockIdx.x;
  SegmentIter it;
  it.u = unit_begin(w, U, G);
  it.u_end = unit_begin(w + 1, U, G);
  it.T = T;
  it.rb_per_b = rb_per_b;
  it.units = units;
  it.nrb = nrb;
  it.rb = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) *hdr = PartitionHeader{U, G, units != nullptr ? 1 : 0};
  if (scorer)
    score_role<DC>(c, it, cache, cache_bstride, qt, rows_pad_b, part_ml, w, headroom, vis, kbuf0, kbuf1, kbuf2,
                   pbuf, votes);
  else
    value_role<DC>(c, it, cache, cache_bstride, part_L, w, vis, kbuf0, kbuf1, kbuf2, pbuf, votes);
}

// fp32 variant: 8 threads per row, 32 rows per workgroup, one workgroup
// sweeps all keys (no key partition).  Scores are reduced over the 8 threads
// with shuffles; the final L is written normalized into slot = row-block.
template <int DC>
__global__ __launch_bounds__(256)
void attend_f32_kernel(const float* __restrict__ cache, int64_t cache_bstride, int n_k,
                       const float* __restrict__ qt, int rows_pad_b, int rb_per_b,
                       float* __restrict__ part_L, Visibility vis) {
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
  // keys [0, kv_row) are visible to this row; the workgroup sweeps to the
  // largest kv of its 32 rows (key 0 is visible to every row)
  const int kv_row = vis.kv_of_row(r, n_k);
  const int kv_wg = vis.kv_max_of_rows(r - rloc, 32, n_k);
  for (int key0 = 0; key0 < kv_wg; key0 += BN) {
    const int nk = min(BN, kv_wg - key0);
    __syncthreads();
    for (int e = tid; e < nk * W; e += 256) sK[e] = cbase[(int64_t)key0 * W + e];
    __syncthreads();
    const int nk_row = min(nk, kv_row - key0);
    for (int k = 0; k < nk_row; ++k) {
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

// units[rb] of a chunk-causal call: exclusive prefix sum over row blocks of
// kSegmentUnits plus the key tiles some row of the block can see (Plan),
// units[nrb] = U.  One workgroup; each thread sums a contiguous run of row
// blocks.
__global__ __launch_bounds__(1024)
void units_kernel(int64_t* __restrict__ units, int nrb, int rb_per_b, int n_k, int bn, Visibility vis) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x, per = (nrb + 1023) / 1024;
  const int r0 = min(nrb, t * per), r1 = min(nrb, r0 + per);
  auto tiles = [&](int rb) {
    return (int64_t)((vis.kv_max_of_block((rb % rb_per_b) * kRowsPerBlock, n_k) + bn - 1) / bn) + kSegmentUnits;
  };
  int64_t sum = 0;
  for (int rb = r0; rb < r1; ++rb) sum += tiles(rb);
  part[t] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan of the per-thread sums
    const int64_t v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - sum;
  for (int rb = r0; rb < r1; ++rb) {
    units[rb] = run;
    run += tiles(rb);
  }
  if (t == 1023) units[nrb] = part[1023];
}

hipError_t launch_units(const Plan& p, const AttendArgs& a, hipStream_t s) {
  int64_t* units = (int64_t*)((char*)a.workspace + p.off_units);
  units_kernel<<<1, 1024, 0, s>>>(units, p.nrb, p.rb_per_b, p.n_k, key_tile(p.d_c), a.vis);
  return hipGetLastError();
}

hipError_t launch_attend_bf16(const Plan& p, const AttendArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  const int64_t* units = p.causal ? (const int64_t*)(ws + p.off_units) : nullptr;
  PartitionHeader* hdr = (PartitionHeader*)(ws + p.off_hdr);
  if (p.causal) {
    const hipError_t e = launch_units(p, a, s);
    if (e != hipSuccess) return e;
  }
  const u16* cache = (const u16*)a.cache;
  const u16* qt = (const u16*)(ws + p.off_qt);
  float* L = (float*)(ws + p.off_L);
  float* ml = (float*)(ws + p.off_ml);
  const dim3 grid(p.G);
  switch (p.d_c) {
    case 64: attend_bf16_kernel<64><<<grid, dim3(attend_waves<64>() * 64), 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom, a.vis, units, p.nrb, hdr); break;
    case 128: attend_bf16_kernel<128><<<grid, dim3(attend_waves<128>() * 64), 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom, a.vis, units, p.nrb, hdr); break;
    case 192: attend_bf16_kernel<192><<<grid, dim3(attend_waves<192>() * 64), 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, ml, p.T, p.U, p.G, a.headroom, a.vis, units, p.nrb, hdr); break;
    case 256: return launch_attend_wide_bf16(p, a, s);   // value accumulators would not fit the role split
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
    case 64: attend_f32_kernel<64><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, a.vis); break;
    case 128: attend_f32_kernel<128><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, a.vis); break;
    case 192: attend_f32_kernel<192><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, a.vis); break;
    case 256: attend_f32_kernel<256><<<grid, block, 0, s>>>(cache, a.cache_bstride, p.n_k, qt, p.rows_pad_b, p.rb_per_b, L, a.vis); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
