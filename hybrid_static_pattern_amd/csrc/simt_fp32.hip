// Hybrid causal attention, float32 storage and arithmetic, one thread per row.
//
// Method: "When Can Attention Heads Be Statically Defined?: 中文精读笔记", part 一 (ordinary
// causal softmax head), part 二.3 Eq. (3) (compact static pattern) and part 二.4 (frozen
// heads mix the current V; their backward is dV = P^T dO only).
//
// This path serves float32 inputs, whose accuracy bar (normwise relative error 1e-5) the
// bf16 matrix cores cannot meet. It favours plain, exact arithmetic (libm exp, exact
// online-softmax rescaling) over speed; the bf16 MFMA kernels carry the workloads.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

constexpr int R = 64;  // rows per block = threads per block

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dO;
  const float* lse_in;
  const float* alpha;
  const float* rho;
  const float* delta;
  float* out;     // O (fwd) / dQ (bwd dq) / dK (bwd dkdv)
  float* out2;    // dV (bwd dkdv)
  float* lse;
  int tab_stride, B, H, T;
  int Hkv, G;                 // key/value heads; query heads per key/value head
  float scale;
  uint8_t frozen[kMaxHeads];  // per head: 1 if frozen
};

// row offset of the key/value head that query head h of batch entry b reads
__device__ __forceinline__ size_t kv_rows(const F32Params& p, int bh, int h) {
  return ((size_t)(bh / p.H) * p.Hkv + h / p.G) * p.T;
}

template <int D>
__global__ __launch_bounds__(R) void fwd_fp32_kernel(const F32Params p) {
  __shared__ float ks[R][D];
  __shared__ float vs[R][D];
  const int tile = blockIdx.x, bh = blockIdx.y, h = bh % p.H;
  const int t = threadIdx.x, i = tile * R + t, T = p.T;
  const bool frz = p.frozen[h] != 0;
  const size_t head = (size_t)bh * T, kvh = kv_rows(p, bh, h);
  float q[D], o[D];
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m = kNegInf, l = 0.f;
  const float* al = p.alpha + (size_t)h * p.tab_stride;
  const float* rh = p.rho + (size_t)h * p.tab_stride;
  if (!frz)
    for (int d = 0; d < D; ++d) q[d] = (i < T) ? p.q[(head + i) * D + d] : 0.f;
  const int jend = min(T, (tile + 1) * R);
  for (int j0 = 0; j0 < jend; j0 += R) {
    __syncthreads();
    for (int x = t; x < R * D; x += R) {
      const int r = x / D, d = x % D, j = j0 + r;
      ks[r][d] = (!frz && j < T) ? p.k[(kvh + j) * D + d] : 0.f;
      vs[r][d] = (j < T) ? p.v[(kvh + j) * D + d] : 0.f;
    }
    __syncthreads();
    if (i >= T) continue;
    for (int r = 0; r < R; ++r) {
      const int j = j0 + r;
      if (j > i) break;
      // logit: scale q.k for an ordinary head, alpha(j) + rho(i - j) for a frozen one (Eq. (3))
      float s;
      if (frz) {
        s = al[j] + rh[i - j];
      } else {
        s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[r][d], s);
        s *= p.scale;
      }
      if (s == kNegInf) continue;  // zero weight
      if (s > m) {
        const float corr = (m == kNegInf) ? 0.f : expf(m - s);
        l *= corr;
        for (int d = 0; d < D; ++d) o[d] *= corr;
        m = s;
      }
      const float w = expf(s - m);
      l += w;
      for (int d = 0; d < D; ++d) o[d] = fmaf(w, vs[r][d], o[d]);
    }
  }
  if (i < T) {
    const float inv = 1.f / l;
    for (int d = 0; d < D; ++d) p.out[(head + i) * D + d] = o[d] * inv;
    p.lse[head + i] = m + logf(l);
  }
}

// dK, dV of ordinary heads and dV of frozen heads: one thread per key, queries i >= j.
template <int D>
__global__ __launch_bounds__(R) void dkdv_fp32_kernel(const F32Params p) {
  __shared__ float qs[R][D];
  __shared__ float gs[R][D];
  __shared__ float ls[R], ds_[R];
  const int tile = blockIdx.x, bh = blockIdx.y, h = bh % p.H;
  const int t = threadIdx.x, j = tile * R + t, T = p.T;
  const bool frz = p.frozen[h] != 0;
  const size_t head = (size_t)bh * T, kvh = kv_rows(p, bh, h);
  const float* al = p.alpha + (size_t)h * p.tab_stride;
  const float* rh = p.rho + (size_t)h * p.tab_stride;
  float kr[D], vr[D], dk[D], dv[D];
  for (int d = 0; d < D; ++d) {
    kr[d] = (!frz && j < T) ? p.k[(kvh + j) * D + d] : 0.f;
    vr[d] = (!frz && j < T) ? p.v[(kvh + j) * D + d] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  for (int i0 = tile * R; i0 < T; i0 += R) {
    __syncthreads();
    for (int x = t; x < R * D; x += R) {
      const int r = x / D, d = x % D, i = i0 + r;
      qs[r][d] = (!frz && i < T) ? p.q[(head + i) * D + d] : 0.f;
      gs[r][d] = (i < T) ? p.dO[(head + i) * D + d] : 0.f;
    }
    if (t < R) {
      const int i = i0 + t;
      ls[t] = (i < T) ? p.lse_in[head + i] : 0.f;
      ds_[t] = (!frz && i < T) ? p.delta[head + i] : 0.f;
    }
    __syncthreads();
    if (j >= T) continue;
    for (int r = 0; r < R; ++r) {
      const int i = i0 + r;
      if (i >= T) break;
      if (i < j) continue;
      if (frz) {
        const float w = expf(al[j] + rh[i - j] - ls[r]);
        for (int d = 0; d < D; ++d) dv[d] = fmaf(w, gs[r][d], dv[d]);
      } else {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(qs[r][d], kr[d], s);
          dp = fmaf(gs[r][d], vr[d], dp);
        }
        const float w = expf(s * p.scale - ls[r]);
        const float dsv = w * (dp - ds_[r]);
        for (int d = 0; d < D; ++d) {
          dv[d] = fmaf(w, gs[r][d], dv[d]);
          dk[d] = fmaf(dsv, qs[r][d], dk[d]);
        }
      }
    }
  }
  if (j < T) {
    for (int d = 0; d < D; ++d) p.out2[(head + j) * D + d] = dv[d];
    if (!frz)
      for (int d = 0; d < D; ++d) p.out[(head + j) * D + d] = dk[d] * p.scale;
  }
}

// dQ of ordinary heads: one thread per query, keys j <= i.
template <int D>
__global__ __launch_bounds__(R) void dq_fp32_kernel(const F32Params p) {
  __shared__ float ks[R][D];
  __shared__ float vs[R][D];
  const int tile = blockIdx.x, bh = blockIdx.y, h = bh % p.H;
  if (p.frozen[h]) return;
  const int t = threadIdx.x, i = tile * R + t, T = p.T;
  const size_t head = (size_t)bh * T, kvh = kv_rows(p, bh, h);
  float q[D], g[D], dq[D];
  for (int d = 0; d < D; ++d) {
    q[d] = (i < T) ? p.q[(head + i) * D + d] : 0.f;
    g[d] = (i < T) ? p.dO[(head + i) * D + d] : 0.f;
    dq[d] = 0.f;
  }
  const float lse = (i < T) ? p.lse_in[head + i] : 0.f;
  const float dl = (i < T) ? p.delta[head + i] : 0.f;
  const int jend = min(T, (tile + 1) * R);
  for (int j0 = 0; j0 < jend; j0 += R) {
    __syncthreads();
    for (int x = t; x < R * D; x += R) {
      const int r = x / D, d = x % D, j = j0 + r;
      ks[r][d] = (j < T) ? p.k[(kvh + j) * D + d] : 0.f;
      vs[r][d] = (j < T) ? p.v[(kvh + j) * D + d] : 0.f;
    }
    __syncthreads();
    if (i >= T) continue;
    for (int r = 0; r < R; ++r) {
      const int j = j0 + r;
      if (j > i) break;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(q[d], ks[r][d], s);
        dp = fmaf(g[d], vs[r][d], dp);
      }
      const float w = expf(s * p.scale - lse);
      const float dsv = w * (dp - dl);
      for (int d = 0; d < D; ++d) dq[d] = fmaf(dsv, ks[r][d], dq[d]);
    }
  }
  if (i < T)
    for (int d = 0; d < D; ++d) p.out[(head + i) * D + d] = dq[d] * p.scale;
}

F32Params base_params(const AttnArgs& a) {
  F32Params p{};
  p.tab_stride = a.tab_stride;
  p.B = a.B;
  p.H = a.H;
  p.T = a.T;
  p.Hkv = a.Hkv;
  p.G = a.G;
  p.scale = a.scale;
  for (int x = 0; x < kMaxHeads; ++x) p.frozen[x] = 0;
  for (int x = 0; x < a.heads.n_frz; ++x) p.frozen[a.heads.frz[x]] = 1;
  return p;
}

}  // namespace

hipError_t launch_fwd_fp32(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const float* alpha, const float* rho, void* o, float* lse,
                           hipStream_t s) {
  F32Params p = base_params(a);
  p.q = static_cast<const float*>(q);
  p.k = static_cast<const float*>(k);
  p.v = static_cast<const float*>(v);
  p.alpha = alpha;
  p.rho = rho;
  p.out = static_cast<float*>(o);
  p.lse = lse;
  dim3 grid((a.T + R - 1) / R, a.B * a.H);
  prof_begin("fwd_fp32", s);
  if (a.D == 64)
    hipLaunchKernelGGL(fwd_fp32_kernel<64>, grid, dim3(R), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_fp32_kernel<128>, grid, dim3(R), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_bwd_fp32(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const float* alpha, const float* rho, float* dq, float* dk,
                           float* dv, float* delta, hipStream_t s) {
  hipError_t e = launch_delta(a, o, dO, delta, lse, nullptr, s);
  if (e != hipSuccess) return e;
  F32Params p = base_params(a);
  p.q = static_cast<const float*>(q);
  p.k = static_cast<const float*>(k);
  p.v = static_cast<const float*>(v);
  p.dO = static_cast<const float*>(dO);
  p.lse_in = lse;
  p.alpha = alpha;
  p.rho = rho;
  p.delta = delta;
  dim3 grid((a.T + R - 1) / R, a.B * a.H);
  p.out = dk;
  p.out2 = dv;
  prof_begin("dkdv_fp32", s);
  if (a.D == 64)
    hipLaunchKernelGGL(dkdv_fp32_kernel<64>, grid, dim3(R), 0, s, p);
  else
    hipLaunchKernelGGL(dkdv_fp32_kernel<128>, grid, dim3(R), 0, s, p);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.heads.n_dyn == 0) return hipSuccess;
  p.out = dq;
  p.out2 = nullptr;
  prof_begin("dq_fp32", s);
  if (a.D == 64)
    hipLaunchKernelGGL(dq_fp32_kernel<64>, grid, dim3(R), 0, s, p);
  else
    hipLaunchKernelGGL(dq_fp32_kernel<128>, grid, dim3(R), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
