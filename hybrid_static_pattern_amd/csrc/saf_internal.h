// Internal interface between the C-ABI layer (saf_api.cpp) and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "saf.h"

namespace saf {

constexpr int kMaxHeads = 256;

// Head lists of one layer: the dynamic (ordinary) heads and the frozen heads (frozen in
// ascending head order; ordinary ones too, except that with shared key/value heads they may
// be dealt out so that each group's heads share an XCD, see validate_attn).
struct HeadLists {
  int n_dyn, n_frz;
  uint8_t dyn[kMaxHeads];
  uint8_t frz[kMaxHeads];
};

struct AttnArgs {
  int B, H, T, D;
  int Hkv, G;           // key/value heads and query heads per key/value head (H = G * Hkv)
  bool bf16;            // io dtype
  float scale;
  int tab_stride;
  HeadLists heads;
};

// Records a thread-local error message (printf format) for saf_last_error and returns st.
saf_status set_error(saf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Kernel timing hooks (saf_prof_*); no-ops unless enabled on this thread.
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

// Forward (ordinary and frozen heads in one launch).
hipError_t launch_fwd_bf16(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const float* alpha, const float* rho, void* o, float* lse,
                           hipStream_t s);
hipError_t launch_fwd_fp32(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const float* alpha, const float* rho, void* o, float* lse,
                           hipStream_t s);

// delta_i = sum_c dO_ic O_ic for ordinary heads, into `delta` [B, H, T] float32, and (if
// ls2 is not null) ls2 = lse * log2(e) for the same rows.
hipError_t launch_delta(const AttnArgs& a, const void* o, const void* dO, float* delta,
                        const float* lse, float* ls2, hipStream_t s);

// Backward workspace: two [B, H, T] float32 arrays (delta, then lse * log2(e)), each padded
// to a multiple of 64 floats; attn_ws_floats is one array's length.
inline size_t attn_ws_floats(const AttnArgs& a) { return ((size_t)a.B * a.H * a.T + 63) / 64 * 64; }
// With shared key/value heads (G > 1) the backward kernels write per-query-head dK and dV
// into two more [B, H, T, D] float32 arrays of the workspace, which launch_gqa_reduce sums
// over each group.
inline size_t gqa_ws_floats(const AttnArgs& a) {
  return a.G > 1 ? ((size_t)a.B * a.H * a.T * a.D + 63) / 64 * 64 : 0;
}
// Frozen heads' dO in float16 for the frozen-head dV product (frz_half.hip): per batch entry b
// and frozen head f, dO[b, frz[f]] scaled by 2^-e_bf and rounded to fp16, [B, n_frz, T, D]; the
// block maxima of the first pass; e_bf [B * n_frz]. Blocks of kFrzBlock values.
constexpr int kFrzBlock = 8192;
struct FrzHalfWs {
  uint16_t* dh;
  float* amax;
  int32_t* dexp;
};
inline int frz_half_blocks(const AttnArgs& a) {
  return (int)(((size_t)a.T * a.D + kFrzBlock - 1) / kFrzBlock);
}
// bytes of the three arrays, each padded to 256 bytes (0 without frozen heads)
inline size_t frz_half_ws_bytes(const AttnArgs& a) {
  if (a.heads.n_frz == 0) return 0;
  const size_t ns = (size_t)a.B * a.heads.n_frz;
  auto pad = [](size_t x) { return (x + 255) / 256 * 256; };
  return pad(ns * a.T * a.D * 2) + pad(ns * frz_half_blocks(a) * 4) + pad(ns * 4);
}
inline FrzHalfWs frz_half_ws(const AttnArgs& a, void* base) {
  const size_t ns = (size_t)a.B * a.heads.n_frz;
  auto pad = [](size_t x) { return (x + 255) / 256 * 256; };
  char* c = static_cast<char*>(base);
  FrzHalfWs w;
  w.dh = reinterpret_cast<uint16_t*>(c);
  c += pad(ns * a.T * a.D * 2);
  w.amax = reinterpret_cast<float*>(c);
  c += pad(ns * frz_half_blocks(a) * 4);
  w.dexp = reinterpret_cast<int32_t*>(c);
  return w;
}
// The block-maxima pass (unless amax_done: the dQ kernel ran it), then the conversion.
hipError_t launch_frz_half(const AttnArgs& a, const void* dO, const FrzHalfWs& ws, bool amax_done,
                           hipStream_t s);
struct FrzAmaxArgs;
FrzAmaxArgs frz_amax_args(const AttnArgs& a, const void* dO, const FrzHalfWs& ws);

hipError_t launch_gqa_reduce(const AttnArgs& a, const float* dk_heads, const float* dv_heads, float* dk,
                             float* dv, hipStream_t s);

// Backward. `delta` is the workspace; `fh` the frozen heads' fp16 dO (launch_frz_half first).
hipError_t launch_bwd_bf16(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const float* alpha, const float* rho, float* dq, float* dk,
                           float* dv, float* delta, const FrzHalfWs& fh, hipStream_t s);
hipError_t launch_bwd_fp32(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const float* alpha, const float* rho, float* dq, float* dk,
                           float* dv, float* delta, hipStream_t s);

// Calibration score.
struct VarArgs {
  int N, H, T, D;
  bool bf16;
  float scale;
};
size_t var_workspace_bytes(const VarArgs& a);
// kl = false: the variance score s_var of Eq. (1); kl = true: the forward-KL score s^KL
// (same A_hat, the score written to s_var and ranked).
hipError_t launch_var_score(const VarArgs& a, const void* q, const void* k, float* a_hat,
                            double* s_var, int32_t* rank, void* ws, hipStream_t s, bool kl);
// Sharp mean pattern [H, T, T] float32 (no workspace).
hipError_t launch_sharp_mean(const VarArgs& a, const void* q, const void* k, float* out, hipStream_t s);

// Compact pattern fit.
// Fit schedules (the values of saf_fit_desc.schedule) and the per-head kernel's limits: it
// keeps a whole head in one workgroup's LDS (T <= kFitHeadMaxT) and is chosen automatically
// for kFitHeadMinHeads heads or more, or for lines of at most kFitHeadShortT. Measured at
// T = 1024 (400 steps): the per-step launches take about 2.7 ms + 0.44 ms per head, the
// per-head kernel 8.1 ms for up to 256 heads (one workgroup per CU), both scaling with T^2
// above their launch costs.
constexpr int kFitAuto = 0, kFitPerStep = 1, kFitPerHead = 2;
constexpr int kFitHeadMaxT = 2048;
constexpr int kFitHeadMinHeads = 16;
constexpr int kFitHeadShortT = 256;
struct FitArgs {
  int H, T, steps;
  float lr, beta1, beta2, eps;
  int schedule;
};
bool fit_per_head(const FitArgs& f);
hipError_t launch_pattern_stats(int H, int T, const float* a, float* col, float* dist, float* ent,
                                hipStream_t s);
hipError_t launch_compact_marginals(int H, int T, const float* alpha, const float* rho, float* logz,
                                    float* col_p, float* dist_p, hipStream_t s);
// Workspace of the fit: log Z, the other alpha and rho buffers, and Adam's m and v for both
// ([H, 2T] each), every array padded to a multiple of 64 floats.
size_t fit_workspace_floats(int H, int T);
hipError_t launch_compact_fit(const FitArgs& f, const float* col, const float* dist, const float* ent,
                              float* alpha, float* rho, float* kl, float* ws, hipStream_t s);

}  // namespace saf
