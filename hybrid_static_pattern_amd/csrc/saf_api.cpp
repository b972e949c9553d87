// libsaf C ABI: argument validation, head lists, workspace layout and kernel dispatch.
// The entry points and their contracts are declared in include/saf.h.
#include "saf.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "saf_internal.h"

namespace {

thread_local std::string g_err;

saf_status vfail(saf_status st, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_err = buf;
  return st;
}

saf_status fail(saf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
saf_status fail(saf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

saf_status hip_fail(hipError_t e, const char* where) {
  return fail(SAF_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------- timing log

struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};

struct ProfState {
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<ProfRec> recs;
  static constexpr size_t kCap = 4096;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void recycle() {
    for (auto& r : recs) {
      pool.push_back(r.start);
      pool.push_back(r.stop);
    }
    recs.clear();
  }
  ~ProfState() {
    recycle();
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

thread_local ProfState g_prof;

saf_status validate_attn(const saf_attn_desc* d, saf::AttnArgs* a) {
  if (!d) return fail(SAF_EINVAL, "desc is NULL");
  if (d->B < 1 || d->H < 1 || d->T < 1)
    return fail(SAF_EINVAL, "B, H, T must be >= 1 (got %d, %d, %d)", d->B, d->H, d->T);
  if (d->D != 64 && d->D != 128) return fail(SAF_EUNSUPPORTED, "D must be 64 or 128 (got %d)", d->D);
  if (d->H > saf::kMaxHeads) return fail(SAF_EUNSUPPORTED, "H must be <= %d (got %d)", saf::kMaxHeads, d->H);
  if (d->io_dtype != SAF_FP32 && d->io_dtype != SAF_BF16) return fail(SAF_EINVAL, "unknown io_dtype %d", (int)d->io_dtype);
  if (d->grad_dtype != SAF_FP32)
    return fail(SAF_EUNSUPPORTED, "grad_dtype must be SAF_FP32 (float32 gradients)");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(SAF_EINVAL, "scale must be finite and > 0");
  if (!d->frozen_mask) return fail(SAF_EINVAL, "frozen_mask is NULL");
  if ((int64_t)d->B * d->H * d->T > (int64_t)1 << 31)
    return fail(SAF_EUNSUPPORTED, "B*H*T must be <= 2^31");
  const int32_t hkv = d->kv_heads == 0 ? d->H : d->kv_heads;
  if (hkv < 1 || hkv > d->H || d->H % hkv != 0)
    return fail(SAF_EINVAL, "kv_heads (%d) must be 0 or a divisor of H (%d)", d->kv_heads, d->H);
  a->B = d->B;
  a->H = d->H;
  a->Hkv = hkv;
  a->G = d->H / hkv;
  a->T = d->T;
  a->D = d->D;
  a->bf16 = d->io_dtype == SAF_BF16;
  a->scale = d->scale;
  a->tab_stride = d->tab_stride;
  a->heads.n_dyn = a->heads.n_frz = 0;
  std::memset(a->heads.dyn, 0, sizeof(a->heads.dyn));
  std::memset(a->heads.frz, 0, sizeof(a->heads.frz));
  for (int h = 0; h < d->H; ++h) {
    if (d->frozen_mask[h]) a->heads.frz[a->heads.n_frz++] = (uint8_t)h;
    else a->heads.dyn[a->heads.n_dyn++] = (uint8_t)h;
  }
  // With shared key/value heads, the ordinary heads of one group should run on one XCD, so
  // that their reads of the group's K and V share that XCD's L2. The attention kernels put
  // ordinary (b, h) stream s = b n_dyn + x on XCD s mod 8; when n_dyn is a multiple of 8
  // that is x mod 8, and dealing the ascending list out in contiguous runs of n_dyn / 8
  // (run c to positions c, c + 8, ...) keeps consecutive heads, hence groups, together.
  const int nd = a->heads.n_dyn;
  if (a->G > 1 && nd % 8 == 0 && nd > 8) {
    uint8_t sorted[saf::kMaxHeads];
    std::memcpy(sorted, a->heads.dyn, sizeof(sorted));
    const int per = nd / 8;
    for (int k = 0; k < nd; ++k) a->heads.dyn[(k % per) * 8 + k / per] = sorted[k];
  }
  if (a->heads.n_frz > 0 && d->tab_stride < d->T)
    return fail(SAF_EINVAL, "tab_stride (%d) must be >= T (%d)", d->tab_stride, d->T);
  return SAF_OK;
}

saf_status check_ptr(const void* p, bool required, const char* name) {
  if (!p) return required ? fail(SAF_EINVAL, "%s is NULL", name) : SAF_OK;
  if (!aligned16(p)) return fail(SAF_EINVAL, "%s is not 16-byte aligned", name);
  return SAF_OK;
}

#define SAF_TRY(x)                       \
  do {                                   \
    saf_status _st = (x);                \
    if (_st != SAF_OK) return _st;       \
  } while (0)

}  // namespace

namespace saf {

saf_status set_error(saf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(st, fmt, ap);
  va_end(ap);
  return st;
}

void prof_begin(const char* name, hipStream_t s) {
  if (!g_prof.on || g_prof.recs.size() >= ProfState::kCap) return;
  ProfRec r{name, g_prof.take(), g_prof.take()};
  if (!r.start || !r.stop) return;
  (void)hipEventRecord(r.start, s);
  g_prof.recs.push_back(r);
}

void prof_end(hipStream_t s) {
  if (!g_prof.on || g_prof.recs.empty()) return;
  (void)hipEventRecord(g_prof.recs.back().stop, s);
}

}  // namespace saf

extern "C" {

saf_status saf_attn_fwd(const saf_attn_desc* desc, const void* q, const void* k, const void* v,
                        const float* alpha, const float* rho, void* o, float* lse, void* stream) {
  saf::AttnArgs a;
  SAF_TRY(validate_attn(desc, &a));
  const bool any_dyn = a.heads.n_dyn > 0, any_frz = a.heads.n_frz > 0;
  SAF_TRY(check_ptr(q, any_dyn, "q"));
  SAF_TRY(check_ptr(k, any_dyn, "k"));
  SAF_TRY(check_ptr(v, true, "v"));
  SAF_TRY(check_ptr(alpha, any_frz, "alpha"));
  SAF_TRY(check_ptr(rho, any_frz, "rho"));
  SAF_TRY(check_ptr(o, true, "o"));
  SAF_TRY(check_ptr(lse, true, "lse"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e = a.bf16 ? saf::launch_fwd_bf16(a, q, k, v, alpha, rho, o, lse, s)
             : saf::launch_fwd_fp32(a, q, k, v, alpha, rho, o, lse, s);
  if (e != hipSuccess) return hip_fail(e, "hybrid forward launch");
  return SAF_OK;
}

size_t saf_attn_workspace_size(const saf_attn_desc* desc) {
  saf::AttnArgs a;
  if (validate_attn(desc, &a) != SAF_OK) return 0;
  return (2 * saf::attn_ws_floats(a) + 2 * saf::gqa_ws_floats(a)) * sizeof(float) +
         (a.bf16 ? saf::frz_half_ws_bytes(a) : 0);
}

saf_status saf_attn_bwd(const saf_attn_desc* desc, const void* q, const void* k, const void* v,
                        const void* o, const void* dO, const float* lse, const float* alpha,
                        const float* rho, void* dq, void* dk, void* dv, void* workspace,
                        size_t ws_bytes, void* stream) {
  saf::AttnArgs a;
  SAF_TRY(validate_attn(desc, &a));
  const bool any_dyn = a.heads.n_dyn > 0, any_frz = a.heads.n_frz > 0;
  SAF_TRY(check_ptr(q, any_dyn, "q"));
  SAF_TRY(check_ptr(k, any_dyn, "k"));
  SAF_TRY(check_ptr(v, any_dyn, "v"));
  SAF_TRY(check_ptr(o, any_dyn, "o"));
  SAF_TRY(check_ptr(dO, true, "dO"));
  SAF_TRY(check_ptr(lse, true, "lse"));
  SAF_TRY(check_ptr(alpha, any_frz, "alpha"));
  SAF_TRY(check_ptr(rho, any_frz, "rho"));
  SAF_TRY(check_ptr(dq, any_dyn, "dq"));
  SAF_TRY(check_ptr(dk, any_dyn, "dk"));
  SAF_TRY(check_ptr(dv, true, "dv"));
  const size_t need = saf_attn_workspace_size(desc);
  SAF_TRY(check_ptr(workspace, need > 0, "workspace"));
  if (ws_bytes < need) return fail(SAF_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  float* delta = static_cast<float*>(workspace);
  // shared key/value heads: per-query-head dK, dV into the workspace, then summed per group
  float* dk_out = static_cast<float*>(dk);
  float* dv_out = static_cast<float*>(dv);
  if (a.G > 1) {
    dk_out = delta + 2 * saf::attn_ws_floats(a);
    dv_out = dk_out + saf::gqa_ws_floats(a);
  }
  // bf16: the frozen heads' dO in fp16 after the float32 arrays (see frz_half.hip)
  saf::FrzHalfWs fh{};
  if (a.bf16) fh = saf::frz_half_ws(a, delta + 2 * saf::attn_ws_floats(a) + 2 * saf::gqa_ws_floats(a));
  hipError_t e = a.bf16 ? saf::launch_bwd_bf16(a, q, k, v, o, dO, lse, alpha, rho, static_cast<float*>(dq),
                                               dk_out, dv_out, delta, fh, s)
                        : saf::launch_bwd_fp32(a, q, k, v, o, dO, lse, alpha, rho, static_cast<float*>(dq),
                                               dk_out, dv_out, delta, s);
  if (e == hipSuccess && a.G > 1)
    e = saf::launch_gqa_reduce(a, dk_out, dv_out, static_cast<float*>(dk), static_cast<float*>(dv), s);
  if (e != hipSuccess) return hip_fail(e, "hybrid backward launch");
  return SAF_OK;
}

static saf_status validate_var(const saf_var_desc* d, saf::VarArgs* a) {
  if (!d) return fail(SAF_EINVAL, "desc is NULL");
  if (d->N < 2) return fail(SAF_EINVAL, "N must be >= 2 (Eq. (1) divides by N - 1), got %d", d->N);
  if (d->H < 1 || d->T < 1) return fail(SAF_EINVAL, "H and T must be >= 1 (got %d, %d)", d->H, d->T);
  if (d->D != 64 && d->D != 128) return fail(SAF_EUNSUPPORTED, "D must be 64 or 128 (got %d)", d->D);
  if (d->H > saf::kMaxHeads) return fail(SAF_EUNSUPPORTED, "H must be <= %d (got %d)", saf::kMaxHeads, d->H);
  if (d->io_dtype != SAF_BF16) return fail(SAF_EUNSUPPORTED, "saf_var_score implements bf16 inputs only");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(SAF_EINVAL, "scale must be finite and > 0");
  if ((int64_t)d->N * d->H * d->T > (int64_t)1 << 31) return fail(SAF_EUNSUPPORTED, "N*H*T must be <= 2^31");
  a->N = d->N;
  a->H = d->H;
  a->T = d->T;
  a->D = d->D;
  a->bf16 = true;
  a->scale = d->scale;
  return SAF_OK;
}

size_t saf_var_workspace_size(const saf_var_desc* desc) {
  saf::VarArgs a;
  if (validate_var(desc, &a) != SAF_OK) return 0;
  return saf::var_workspace_bytes(a);
}

saf_status saf_var_score(const saf_var_desc* desc, const void* q, const void* k, float* a_hat,
                         double* s_var, int32_t* rank, void* workspace, size_t ws_bytes,
                         void* stream) {
  saf::VarArgs a;
  SAF_TRY(validate_var(desc, &a));
  SAF_TRY(check_ptr(q, true, "q"));
  SAF_TRY(check_ptr(k, true, "k"));
  SAF_TRY(check_ptr(a_hat, true, "a_hat"));
  SAF_TRY(check_ptr(s_var, true, "s_var"));
  SAF_TRY(check_ptr(rank, true, "rank"));
  SAF_TRY(check_ptr(workspace, true, "workspace"));
  const size_t need = saf::var_workspace_bytes(a);
  if (ws_bytes < need) return fail(SAF_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  (void)hipGetLastError();
  hipError_t e = saf::launch_var_score(a, q, k, a_hat, s_var, rank, workspace, static_cast<hipStream_t>(stream), false);
  if (e != hipSuccess) return hip_fail(e, "var_score launch");
  return SAF_OK;
}

saf_status saf_kl_score(const saf_var_desc* desc, const void* q, const void* k, float* a_hat, double* s_kl,
                        int32_t* rank, void* workspace, size_t ws_bytes, void* stream) {
  saf::VarArgs a;
  SAF_TRY(validate_var(desc, &a));
  SAF_TRY(check_ptr(q, true, "q"));
  SAF_TRY(check_ptr(k, true, "k"));
  SAF_TRY(check_ptr(a_hat, true, "a_hat"));
  SAF_TRY(check_ptr(s_kl, true, "s_kl"));
  SAF_TRY(check_ptr(rank, true, "rank"));
  SAF_TRY(check_ptr(workspace, true, "workspace"));
  const size_t need = saf::var_workspace_bytes(a);
  if (ws_bytes < need) return fail(SAF_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  (void)hipGetLastError();
  hipError_t e = saf::launch_var_score(a, q, k, a_hat, s_kl, rank, workspace, static_cast<hipStream_t>(stream), true);
  if (e != hipSuccess) return hip_fail(e, "kl_score launch");
  return SAF_OK;
}

saf_status saf_sharp_mean(const saf_var_desc* desc, const void* q, const void* k, float* p_sharp, void* stream) {
  saf::VarArgs a;
  SAF_TRY(validate_var(desc, &a));
  SAF_TRY(check_ptr(q, true, "q"));
  SAF_TRY(check_ptr(k, true, "k"));
  SAF_TRY(check_ptr(p_sharp, true, "p_sharp"));
  (void)hipGetLastError();
  hipError_t e = saf::launch_sharp_mean(a, q, k, p_sharp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sharp_mean launch");
  return SAF_OK;
}

int32_t saf_select_heads(const double* s_var_all, int32_t n_heads, double r, int32_t* out) {
  if (!s_var_all || !out || n_heads < 1 || !(r >= 0.0 && r <= 1.0)) {
    fail(SAF_EINVAL, "saf_select_heads: bad arguments");
    return -1;
  }
  std::vector<int32_t> idx(n_heads);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return s_var_all[x] < s_var_all[y]; });
  const int32_t kk = (int32_t)std::floor(r * n_heads + 0.5);
  for (int32_t x = 0; x < kk; ++x) out[x] = idx[x];
  return kk;
}

static saf_status validate_fit_shape(int32_t H, int32_t T) {
  if (H < 1 || T < 1) return fail(SAF_EINVAL, "H and T must be >= 1 (got %d, %d)", H, T);
  if (H > 65535) return fail(SAF_EUNSUPPORTED, "H must be <= 65535 (got %d)", H);
  if ((int64_t)H * T > (int64_t)1 << 31) return fail(SAF_EUNSUPPORTED, "H*T must be <= 2^31");
  return SAF_OK;
}

saf_status saf_pattern_stats(int32_t H, int32_t T, const float* a, float* col, float* dist, float* ent,
                             void* stream) {
  SAF_TRY(validate_fit_shape(H, T));
  SAF_TRY(check_ptr(a, true, "a"));
  SAF_TRY(check_ptr(col, true, "col"));
  SAF_TRY(check_ptr(dist, true, "dist"));
  SAF_TRY(check_ptr(ent, true, "ent"));
  (void)hipGetLastError();
  hipError_t e = saf::launch_pattern_stats(H, T, a, col, dist, ent, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pattern statistics launch");
  return SAF_OK;
}

saf_status saf_compact_marginals(int32_t H, int32_t T, const float* alpha, const float* rho, float* logz,
                                 float* col, float* dist, void* stream) {
  SAF_TRY(validate_fit_shape(H, T));
  SAF_TRY(check_ptr(alpha, true, "alpha"));
  SAF_TRY(check_ptr(rho, true, "rho"));
  SAF_TRY(check_ptr(logz, true, "logz"));
  SAF_TRY(check_ptr(col, true, "col"));
  SAF_TRY(check_ptr(dist, true, "dist"));
  (void)hipGetLastError();
  hipError_t e = saf::launch_compact_marginals(H, T, alpha, rho, logz, col, dist, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compact marginals launch");
  return SAF_OK;
}

static saf_status validate_fit(const saf_fit_desc* d, saf::FitArgs* f) {
  if (!d) return fail(SAF_EINVAL, "desc is NULL");
  SAF_TRY(validate_fit_shape(d->H, d->T));
  if (d->steps < 0) return fail(SAF_EINVAL, "steps must be >= 0 (got %d)", d->steps);
  if (!(d->lr > 0.f) || !std::isfinite(d->lr)) return fail(SAF_EINVAL, "lr must be finite and > 0");
  if (!(d->beta1 >= 0.f && d->beta1 < 1.f) || !(d->beta2 >= 0.f && d->beta2 < 1.f))
    return fail(SAF_EINVAL, "beta1 and beta2 must lie in [0, 1)");
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return fail(SAF_EINVAL, "eps must be finite and >= 0");
  if (d->schedule < saf::kFitAuto || d->schedule > saf::kFitPerHead)
    return fail(SAF_EINVAL, "schedule must be SAF_FIT_AUTO, SAF_FIT_PER_STEP or SAF_FIT_PER_HEAD (got %d)",
                d->schedule);
  if (d->schedule == saf::kFitPerHead && d->T > saf::kFitHeadMaxT)
    return fail(SAF_EUNSUPPORTED, "SAF_FIT_PER_HEAD needs T <= %d (got %d)", saf::kFitHeadMaxT, d->T);
  *f = saf::FitArgs{d->H, d->T, d->steps, d->lr, d->beta1, d->beta2, d->eps, d->schedule};
  return SAF_OK;
}

size_t saf_fit_workspace_size(const saf_fit_desc* desc) {
  saf::FitArgs f;
  if (validate_fit(desc, &f) != SAF_OK) return 0;
  return saf::fit_workspace_floats(f.H, f.T) * sizeof(float);
}

saf_status saf_compact_fit(const saf_fit_desc* desc, const float* col, const float* dist, const float* ent,
                           float* alpha, float* rho, float* kl, void* workspace, size_t ws_bytes,
                           void* stream) {
  saf::FitArgs f;
  SAF_TRY(validate_fit(desc, &f));
  SAF_TRY(check_ptr(col, true, "col"));
  SAF_TRY(check_ptr(dist, true, "dist"));
  SAF_TRY(check_ptr(ent, true, "ent"));
  SAF_TRY(check_ptr(alpha, true, "alpha"));
  SAF_TRY(check_ptr(rho, true, "rho"));
  SAF_TRY(check_ptr(kl, true, "kl"));
  SAF_TRY(check_ptr(workspace, true, "workspace"));
  const size_t need = saf::fit_workspace_floats(f.H, f.T) * sizeof(float);
  if (ws_bytes < need) return fail(SAF_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  (void)hipGetLastError();
  hipError_t e = saf::launch_compact_fit(f, col, dist, ent, alpha, rho, kl, static_cast<float*>(workspace),
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "compact fit launch");
  return SAF_OK;
}

int32_t saf_select_fitted(const double* s_var_all, const float* kl_all, int32_t n_heads, double r,
                          float max_kl, int32_t* out) {
  if (!s_var_all || !kl_all || !out || n_heads < 1 || !(r >= 0.0 && r <= 1.0) || std::isnan(max_kl)) {
    fail(SAF_EINVAL, "saf_select_fitted: bad arguments");
    return -1;
  }
  std::vector<int32_t> idx(n_heads);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) { return s_var_all[x] < s_var_all[y]; });
  const int32_t kk = (int32_t)std::floor(r * n_heads + 0.5);
  int32_t kept = 0;
  for (int32_t x = 0; x < n_heads && kept < kk; ++x)
    if (kl_all[idx[x]] <= max_kl) out[kept++] = idx[x];
  return kept;
}

const char* saf_status_string(saf_status st) {
  switch (st) {
    case SAF_OK: return "SAF_OK";
    case SAF_EINVAL: return "SAF_EINVAL: invalid argument";
    case SAF_EUNSUPPORTED: return "SAF_EUNSUPPORTED: unsupported shape or dtype";
    case SAF_EWORKSPACE: return "SAF_EWORKSPACE: workspace too small";
    case SAF_EHIP: return "SAF_EHIP: HIP runtime error";
  }
  return "unknown saf_status";
}

const char* saf_last_error(void) { return g_err.c_str(); }

saf_status saf_prof_enable(int enable) {
  g_prof.recycle();
  g_prof.on = enable != 0;
  return SAF_OK;
}

int32_t saf_prof_read(const char** names, float* ms, int32_t cap) {
  int32_t n = 0;
  for (auto& r : g_prof.recs) {
    if (n >= cap) break;
    float t = -1.f;
    if (hipEventSynchronize(r.stop) == hipSuccess) (void)hipEventElapsedTime(&t, r.start, r.stop);
    if (names) names[n] = r.name;
    if (ms) ms[n] = t;
    ++n;
  }
  g_prof.recycle();
  return n;
}

}  // extern "C"
