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
