// Launchers of the HIP kernels; the C ABI layer validates arguments and calls these.
#pragma once

#include "mla_common.h"

namespace mla {

struct AppendArgs {
  int batch, n_new, d_model, d_c, d_r, cap, off;
  const void* x;
  const void* w_dkv;
  const void* w_kr;
  const int* pos;
  void* cache;
  RopeSpec rope;
};

struct AbsorbArgs {
  const void* q;
  const void* q_r;
  const int* q_pos;
  const void* w_uk;
  float qscale;   // softmax_scale * log2(e)
  void* qt;       // workspace + plan.off_qt
  RopeSpec rope;
};

struct AttendArgs {
  const void* cache;
  int64_t cache_bstride;  // elements between samples (capacity * width)
  void* workspace;
  float headroom;         // log2 headroom of the single-pass softmax (see attend.hip)
  Visibility vis;         // chunk-causal key limits per query
};

struct UpprojArgs {
  const void* w_uv;
  void* out;
  bool out_f32;
  void* workspace;
};

// ---------------------------------------------------------------------------
// Standard attention over per-head keys and values (attend_mha.hip): the
// dense K/V baseline and the non-absorbed latent form.  bf16 inputs, head_dim
// and value width 128, query/key width dqk = 128 (dense) or 160 (latent:
// d_h + d_r).  Rows are padded per (batch, head) to 256-row blocks.
// ---------------------------------------------------------------------------
struct MhaPlan {
  int32_t B, H, n_q, n_k, dqk;
  int32_t rb_per_bh, rows_pad_h;   // row blocks and padded rows per (batch, head)
  int64_t nrb;                     // B * H * rb_per_bh
  int32_t T;                       // 32-key tiles
  int64_t U;                       // units nrb * T
  int32_t G;                       // attention workgroups
  // byte offsets inside the workspace: scaled queries, partial states,
  // and (non-absorbed form) the materialised per-head K [B, H, n_k, dqk] and V [B, H, n_k, 128]
  int64_t off_qt, off_L, off_ml, off_k, off_v, total;
};

MhaPlan make_mha_plan(int B, int H, int n_q, int n_k, int dqk, bool expanded);

struct MhaQueryArgs {
  const void* q;        // [B, n_q, H, 128]
  const void* q_r;      // [B, n_q, H, dqk - 128] (dqk = 160), else unused
  const int* q_pos;     // [n_q, 3] (dqk = 160), else unused
  RopeSpec rope;
  void* workspace;
};

struct MhaUpliftArgs {
  const void* cache;    // [B, cap, d_c + 32]
  int64_t cap;
  int d_c;
  const void* w_uk;     // [H, 128, d_c]
  const void* w_uv;     // [H, 128, d_c]
  void* workspace;
};

struct MhaAttendArgs {
  const void* k;        // [B, cap, H, dqk], or [B, H, cap, dqk] when head_major
  const void* v;        // [B, cap, H, 128], or [B, H, cap, 128] when head_major
  int64_t cap;
  bool head_major;      // keys of one (batch, head) contiguous (the materialised non-absorbed K and V)
  float headroom;
  float qscale;         // softmax_scale * log2(e), applied to the fp32 scores
  void* out;            // [B, n_q, H, 128]
  bool out_f32;
  void* workspace;
};

hipError_t launch_mha_prep_q(const MhaPlan& p, const MhaQueryArgs& a, hipStream_t s);
hipError_t launch_mha_uplift(const MhaPlan& p, const MhaUpliftArgs& a, hipStream_t s);
hipError_t launch_mha_attend(const MhaPlan& p, const MhaAttendArgs& a, hipStream_t s);

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_f32(const AppendArgs& a, hipStream_t s);
hipError_t launch_absorb_bf16(const Plan& p, const AbsorbArgs& a, hipStream_t s);
hipError_t launch_absorb_f32(const Plan& p, const AbsorbArgs& a, hipStream_t s);
hipError_t launch_attend_bf16(const Plan& p, const AttendArgs& a, hipStream_t s);
hipError_t launch_attend_wide_bf16(const Plan& p, const AttendArgs& a, hipStream_t s);   // d_c = 256
hipError_t launch_attend_f32(const Plan& p, const AttendArgs& a, hipStream_t s);
hipError_t launch_upproj_bf16(const Plan& p, const UpprojArgs& a, hipStream_t s);
hipError_t launch_upproj_f32(const Plan& p, const UpprojArgs& a, hipStream_t s);

}  // namespace mla
