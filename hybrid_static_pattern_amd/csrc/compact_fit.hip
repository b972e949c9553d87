// Compact static pattern fit (web page "When Can Attention Heads Be Statically Defined?:
// 中文精读笔记", part 二.3, Eq. (3), Eq. (4), Appendix A.2).
//
// A candidate head's target pattern A (its mean attention) is replaced by
//   P(i,j) = exp(alpha(j) + rho(i-j)) / Z(i),  j <= i,
// fitted by minimising the mean row cross-entropy of P relative to A. That objective
// depends on A only through its key-position marginal col(j) = sum_i A(i,j) and its
// distance marginal dist(d) = sum_i A(i,i-d) (Eq. (4)):
//   CE = (1/T) [sum_i log Z(i) - sum_j alpha(j) col(j) - sum_d rho(d) dist(d)],
// with gradient (colP(j) - col(j)) / T and (distP(d) - dist(d)) / T, where colP and distP
// are the same marginals of P. Each Adam step therefore needs log Z(i) for every row, then
// both marginals of P; the mean row KL reported at the end is CE minus the target's mean
// row entropy, whose per-column shares the statistics pass also produces.
//
// The per-step kernels give each wave two outputs (rows, columns or distances) and spread
// the sum over an output's line of the causal triangle across the 64 lanes; the 32 outputs
// of a workgroup are consecutive, so the stretch of alpha, rho or log Z their lines read is
// staged in LDS once for the workgroup and read there as consecutive floats. The work per
// step (1.5 T(T+1) exps per head) is spread over 1.5 T waves per head instead of T threads.
// Exponents are shifted by the row's max (log Z) or are never positive (the marginals, since
// log Z(i) bounds every logit of row i), so no exp overflows.
#include <hip/hip_runtime.h>

#include <cmath>

#include "saf_internal.h"

namespace saf {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;
constexpr int LW = 16;     // waves per workgroup in the per-line kernels
constexpr int OPW = 2;     // outputs (rows, columns or distances) per wave in the per-line kernels
constexpr int SW = 16;     // waves per workgroup in the statistics kernel
constexpr int C = 2048;    // keys (or terms) per LDS chunk in the per-line kernels
constexpr int U2 = 2;      // 16-byte reads per lane and table before use in the per-line kernels
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Eq. (4) statistics of the target A [H, T, T] (entries above the diagonal are not read):
// col(x), dist(x) and ent(x) = -sum_{i>=x} A(i,x) log A(i,x) for x = 64 blockIdx.x + lane.
// Wave w sums rows i = x0 + w, x0 + w + SW, ...; row i reads A(i, x) and A(i, i - x), both
// 64 consecutive floats. The SW partial sums are added in a fixed order.
__global__ __launch_bounds__(64 * SW) void stats_kernel(int T, const float* __restrict__ a,
                                                        float* __restrict__ col,
                                                        float* __restrict__ dist,
                                                        float* __restrict__ ent) {
  __shared__ float part[3][SW][64];
  const int h = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x0 = blockIdx.x * 64, x = x0 + lane;
  const float* ah = a + (size_t)h * T * T;
  float c = 0.f, g = 0.f, e = 0.f;
  for (int i = x0 + w; i < T; i += SW) {
    if (x <= i) {
      const float* row = ah + (size_t)i * T;
      const float v = row[x];
      c += v;
      if (v > 0.f) e -= v * logf(v);
      g += row[i - x];
    }
  }
  part[0][w][lane] = c;
  part[1][w][lane] = g;
  part[2][w][lane] = e;
  __syncthreads();
  if (w < 3 && x < T) {
    float s = 0.f;
    for (int u = 0; u < SW; ++u) s += part[w][u][lane];
    float* out = w == 0 ? col : (w == 1 ? dist : ent);
    out[(size_t)h * T + x] = s;
  }
}

// log Z(i) = log sum_{j<=i} exp(alpha(j) + rho(i-j)) for the OPW LW rows of a block, OPW per
// wave (rows i0 + w + LW r). The rows share their keys: chunks of C keys of alpha, and the
// window of rho the rows need for them (C + OPW LW - 1 distances), are staged in LDS once for
// the block, in log2 units. A lane takes 4 consecutive keys per 16-byte read of each table:
// the 4 distances of 4 consecutive keys are consecutive too, but where they start depends on
// the row, so the rho window is staged 4 times, shifted by 0..3 entries, and each row reads
// the copy that makes its reads 16-byte aligned. Each lane keeps its own running max and sum
// (one rescale per group of 4 U2 keys); the lanes are combined once per row.
__global__ __launch_bounds__(64 * LW) void logz_kernel(int T, const float* __restrict__ alpha,
                                                       const float* __restrict__ rho,
                                                       float* __restrict__ logz) {
  constexpr int NR = OPW * LW;   // rows per block
  constexpr int GK = 256 * U2;   // keys per group (4 per lane and read)
  __shared__ float4 sal[C / 4];
  __shared__ __attribute__((aligned(16))) float srh[4][C + NR + 4];
  const int h = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i0 = blockIdx.x * NR;
  const int i_last = min(i0 + NR, T) - 1;
  const float* al = alpha + (size_t)h * T;
  const float* rh = rho + (size_t)h * T;
  float mx[OPW], s[OPW];
#pragma unroll
  for (int r = 0; r < OPW; ++r) {
    mx[r] = kNegInf;
    s[r] = 0.f;
  }
  for (int j0 = 0; j0 <= i_last; j0 += C) {
    __syncthreads();   // the previous chunk is no longer read
    // sal = alpha(j0 + y); copy c of the window: srh[c][y] = rho(d) with
    // d = i0 - j0 - C + 1 + y + c, so that row i and key j read position (i - i0) + C - 1 - (j - j0) - c.
    // All of a thread's loads are issued before the first store, so the block waits for
    // memory once per chunk.
    float* sa = reinterpret_cast<float*>(sal);
    constexpr int NY = (C + NR + 3 + 64 * LW - 1) / (64 * LW);
    float va[NY], vr[NY];
#pragma unroll
    for (int q = 0; q < NY; ++q) {
      const int y = threadIdx.x + 64 * LW * q, d = i0 - j0 - C + 1 + y;
      va[q] = (y < C && j0 + y <= i_last) ? al[j0 + y] : 0.f;
      vr[q] = (y < C + NR + 3 && d >= 0 && d < T) ? rh[d] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NY; ++q) {
      const int y = threadIdx.x + 64 * LW * q;
      if (y < C) sa[y] = va[q] * kLog2e;
      if (y < C + NR + 3) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (y - c >= 0) srh[c][y - c] = vr[q] * kLog2e;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < OPW; ++r) {
      const int i = i0 + w + LW * r;
      if (i > i_last) continue;
      const int c = (i - i0) & 3;
      // keys k .. k + 3 (k a multiple of 4) read rho at positions yl .. yl + 3 of copy c,
      // yl = (i - i0) + C - 4 - k - c, in reverse key order
      const float* rw = srh[c] + (i - i0) + C - 4 - c;
      for (int k0 = 0; k0 < C && j0 + k0 <= i; k0 += GK) {
        float x[4 * U2];
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          const int k = k0 + 256 * u + 4 * lane;
          const float4 av = sal[k >> 2];
          const float4 rv = *reinterpret_cast<const float4*>(rw - k);
          x[4 * u + 0] = av.x + rv.w;
          x[4 * u + 1] = av.y + rv.z;
          x[4 * u + 2] = av.z + rv.y;
          x[4 * u + 3] = av.w + rv.x;
          if (j0 + k0 + GK - 1 > i) {   // the row ends in this group: mask keys past it
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j0 + k + e > i) x[4 * u + e] = kNegInf;
          }
        }
        float cm = x[0];
#pragma unroll
        for (int e = 1; e < 4 * U2; ++e) cm = fmaxf(cm, x[e]);
        if (cm == kNegInf) continue;   // no key of this group for this lane
        const float m_new = fmaxf(mx[r], cm);
        float cs = 0.f;
#pragma unroll
        for (int e = 0; e < 4 * U2; ++e) cs += __builtin_amdgcn_exp2f(x[e] - m_new);
        s[r] = s[r] * __builtin_amdgcn_exp2f(mx[r] - m_new) + cs;
        mx[r] = m_new;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < OPW; ++r) {
    const int i = i0 + w + LW * r;
    if (i > i_last) continue;
    const float m_row = wave_max(mx[r]);   // finite: lane 0 holds key 0
    const float sr = wave_sum(mx[r] == kNegInf ? 0.f : s[r] * __builtin_amdgcn_exp2f(mx[r] - m_row));
    if (lane == 0) logz[(size_t)h * T + i] = (m_row + __log2f(sr)) * kLn2;
  }
}

struct AdamStep {
  float lr, beta1, beta2, eps;
  float bc1, bc2;      // 1 - beta1^t, 1 - beta2^t
  float inv_t;         // 1 / T
};

// Marginals of P. Blocks [0, nb) take columns x (own = alpha(x), other = rho), blocks
// [nb, 2 nb) distances x (own = rho(x), other = alpha), OPW LW consecutive x per block, OPW
// per wave (x0 + w + LW r). Both are S(x) = sum_{t=0}^{T-1-x} exp(other(t) + own(x) - log Z(x + t));
// chunks of C values of `other` and the C + OPW LW - 1 values of log Z the block's outputs
// need are staged in LDS once for the block, in log2 units, log Z 4 times shifted by 0..3 so
// that every output reads it 16 bytes at a time (4 consecutive t per read, as for `other`).
// ADAM = false writes S into colP / distP. ADAM = true takes one Adam step on own(x) with
// gradient (S - target(x)) / T and writes the new value to the other parameter buffer (the
// current values are still being read by other blocks); m and v are [H, 2T], the alpha part
// first. Adam's operands are read before the sums so that their latency overlaps the staging.
template <bool ADAM>
__global__ __launch_bounds__(64 * LW) void marg_kernel(int T, int nb, const float* __restrict__ alpha,
                                                       const float* __restrict__ rho,
                                                       const float* __restrict__ logz,
                                                       float* __restrict__ out_col,    // colP, or new alpha
                                                       float* __restrict__ out_dist,   // distP, or new rho
                                                       const float* __restrict__ col,
                                                       const float* __restrict__ dist,
                                                       float* __restrict__ m, float* __restrict__ v,
                                                       AdamStep st) {
  constexpr int NX = OPW * LW;   // outputs per block
  constexpr int GK = 256 * U2;   // terms per group (4 per lane and read)
  __shared__ float4 soth[C / 4];
  __shared__ __attribute__((aligned(16))) float slz[4][C + NX + 4];
  const int h = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool is_col = (int)blockIdx.x < nb;
  const int x0 = (is_col ? blockIdx.x : blockIdx.x - nb) * NX;
  const size_t hb = (size_t)h * T;
  const float* own = (is_col ? alpha : rho) + hb;
  const float* oth = (is_col ? rho : alpha) + hb;
  const float* lz = logz + hb;
  float ox[OPW], s[OPW], tg[OPW], mo[OPW], vo[OPW];
#pragma unroll
  for (int r = 0; r < OPW; ++r) {
    const int x = x0 + w + LW * r;
    ox[r] = x < T ? own[x] : 0.f;
    s[r] = 0.f;
    if constexpr (ADAM) {
      if (lane == 0 && x < T) {
        const size_t k = (size_t)h * 2 * T + (is_col ? x : T + x);
        tg[r] = (is_col ? col : dist)[hb + x];
        mo[r] = m[k];
        vo[r] = v[k];
      }
    }
  }
  for (int t0 = 0; t0 < T - x0; t0 += C) {
    __syncthreads();   // the previous chunk is no longer read
    // soth = other(t0 + y); copy c: slz[c][y] = log Z(x0 + t0 + y + c); loads first, as in
    // logz_kernel
    float* so = reinterpret_cast<float*>(soth);
    constexpr int NY = (C + NX + 3 + 64 * LW - 1) / (64 * LW);
    float ov[NY], lv[NY];
#pragma unroll
    for (int q = 0; q < NY; ++q) {
      const int y = threadIdx.x + 64 * LW * q;
      ov[q] = (y < C && t0 + y < T) ? oth[t0 + y] : 0.f;
      lv[q] = (y < C + NX + 3 && x0 + t0 + y < T) ? lz[x0 + t0 + y] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < NY; ++q) {
      const int y = threadIdx.x + 64 * LW * q;
      if (y < C) so[y] = ov[q] * kLog2e;
      if (y < C + NX + 3) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (y - c >= 0) slz[c][y - c] = lv[q] * kLog2e;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < OPW; ++r) {
      const int x = x0 + w + LW * r;
      const float o2 = ox[r] * kLog2e;
      const int c = (x - x0) & 3;
      const float* lw = slz[c] + (x - x0) - c;   // log Z(x + t0 + k) = lw[k], 16-byte aligned for k % 4 == 0
      const int n_t = min(C, T - x - t0);        // terms of this chunk for output x
      for (int k0 = 0; k0 < n_t; k0 += GK) {
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          const int k = k0 + 256 * u + 4 * lane;
          const float4 ov = soth[k >> 2];
          const float4 zv = *reinterpret_cast<const float4*>(lw + k);
          float e[4] = {ov.x + o2 - zv.x, ov.y + o2 - zv.y, ov.z + o2 - zv.z, ov.w + o2 - zv.w};
          if (k0 + GK > n_t) {   // the line ends in this group
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (k + q >= n_t) e[q] = kNegInf;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) s[r] += __builtin_amdgcn_exp2f(e[q]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < OPW; ++r) {
    const int x = x0 + w + LW * r;
    if (x >= T) continue;
    const float sum = wave_sum(s[r]);
    if (lane != 0) continue;
    float* out = (is_col ? out_col : out_dist) + hb;
    if constexpr (!ADAM) {
      out[x] = sum;
    } else {
      const float g = (sum - tg[r]) * st.inv_t;
      const size_t k = (size_t)h * 2 * T + (is_col ? x : T + x);
      const float mm = st.beta1 * mo[r] + (1.f - st.beta1) * g;
      const float vv = st.beta2 * vo[r] + (1.f - st.beta2) * g * g;
      m[k] = mm;
      v[k] = vv;
      out[x] = ox[r] - st.lr * (mm / st.bc1) / (sqrtf(vv / st.bc2) + st.eps);
    }
  }
}

// Mean row KL of each head: (1/T) [sum_i log Z(i) - sum_j alpha(j) col(j)
// - sum_d rho(d) dist(d) - sum_j ent(j)], summed in double (the terms are O(T) and cancel).
__global__ __launch_bounds__(256) void kl_kernel(int T, const float* __restrict__ alpha,
                                                 const float* __restrict__ rho,
                                                 const float* __restrict__ logz,
                                                 const float* __restrict__ col,
                                                 const float* __restrict__ dist,
                                                 const float* __restrict__ ent,
                                                 float* __restrict__ kl) {
  __shared__ double part[4];
  const int h = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t hb = (size_t)h * T;
  double acc = 0.0;
  for (int x = threadIdx.x; x < T; x += 256)
    acc += (double)logz[hb + x] - (double)alpha[hb + x] * col[hb + x] -
           (double)rho[hb + x] * dist[hb + x] - (double)ent[hb + x];
  acc = wave_sum(acc);
  if (lane == 0) part[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) kl[h] = (float)((part[0] + part[1] + part[2] + part[3]) / T);
}

__global__ void fill_kernel(float* __restrict__ p, size_t n, float val) {
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x)
    p[x] = val;
}

__global__ void copy_kernel(float* __restrict__ dst, const float* __restrict__ src, size_t n) {
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (size_t)gridDim.x * blockDim.x)
    dst[x] = src[x];
}

// ---------------------------------------------------------------- one workgroup per head
//
// The whole fit of one head in one workgroup of 16 waves, its state in LDS: the parameters
// (natural units), Adam's moments, the targets, the tables derived from the parameters at
// the start of each step, and log Z. A step is four phases separated by barriers (ranges of
// the parameters, tables, log Z, marginals with the Adam update), with no launch and no
// round trip through memory between them. Used when there are enough heads to occupy the
// CUs, or for short lines (the per-step launches spread one head over many CUs instead).
//
// Factored terms. A term of log Z(i) or of a marginal is exp(alpha(j) + rho(i-j) - log Z(i)),
// a product of one factor per table. With A(j) = exp2(alpha2(j) - max alpha2), R(d) =
// exp2(rho2(d) - max rho2) (log2 units) and Zi(i) = exp2(max alpha2 + max rho2 - log2 Z(i)):
//   log2 Z(i) = max alpha2 + max rho2 + log2 sum_{j<=i} A(j) R(i-j),  Zi(i) = 1 / that sum,
//   colP(x)   = A(x) sum_t R(t) Zi(x+t),   distP(d) = R(d) sum_t A(t) Zi(d+t),
// one fused multiply-add per term and no exp. This is exact up to rounding as long as no
// factor or partial product leaves float32's normal range: with spreads (max - min, log2
// units) sa of alpha and sr of rho, A R >= 2^-(sa+sr), Zi >= 1/T, R(t) Zi(x+t) <= 2^sa and
// A(t) Zi(d+t) <= 2^sr (log Z(i) bounds each of its own terms), so sa + sr <= 96 keeps every
// value within [2^-107, 2^96]. A step whose parameters spread further takes the exp path:
// exponents shifted by the row's running max (log Z) or never positive (marginals).
//
// Both phases give each 16-lane group G consecutive rows (or outputs) and each lane 8
// consecutive keys (or terms) at a time: the 8 G terms a lane forms per iteration come from
// 2 16-byte LDS reads of one table and (G + 8) / 4 of the other, whose G + 7 entries cover
// the sums of the two indices, and the reductions stay within 16-lane DPP rows. The
// factored path, one FMA per term, takes G = 8 (1.5 bytes of LDS per term, which then bounds
// it); the exp path G = 4 (2.5 bytes per term), its exps bounding it.
//
// Table padding replaces masks: factors are 0 outside their index range; on the exp path rho
// has -inf before distance 0 and past T - 1, log Z +inf past row T - 1, alpha 0 past T - 1
// (only ever added to a -inf), so no sum of two infinities of opposite sign arises.
constexpr int HW = 16;            // waves per workgroup
constexpr int RPAD = 8;           // entries before distance 0
constexpr int TPAD = 32;          // entries past T - 1 in each table
constexpr float kFactorSpread = 96.f;   // log2 units

struct AdamHyper {
  float lr, beta1, beta2, eps;
};

// v[lane % 16] for the first N lanes of each 16-lane row: spreads the per-row results that
// every lane of the row holds after a reduction over the row's lanes, one per lane.
template <int N>
__device__ __forceinline__ float pick(const float (&v)[N], int i) {
  float r = v[0];
#pragma unroll
  for (int c = 1; c < N; ++c) r = i == c ? v[c] : r;
  return r;
}

// Reductions over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15), every lane getting
// the result: the quad permutations [1,0,3,2] and [2,3,0,1] combine lanes within quads, the
// half-row mirror (lane l <-> 7 - l in each 8) pairs the two quads of a half, the row mirror
// (l <-> 15 - l) the two halves.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  return x + dpp_mov<0x140>(x);
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  return fmaxf(x, dpp_mov<0x140>(x));
}

// The factored tables keep 4 floats of padding after every 64 entries (entry i at
// i + 4 (i / 64)): the lane groups read at 8-float strides, which would otherwise put lanes
// l and l + 8 of one hardware read group on the same LDS banks.
__device__ __forceinline__ int padx(int i) { return i + ((i >> 6) << 2); }
constexpr int padded(int n) { return n + (n + 63) / 64 * 4; }

template <int TMAX>
struct HeadFit {
  float a2[TMAX + TPAD];            // exp path: alpha * log2(e)
  float r2[RPAD + TMAX + TPAD];     // exp path: rho * log2(e), rho(d) at RPAD + d
  float fa[padded(TMAX + TPAD)];          // factored: A (padded layout)
  float fr[padded(RPAD + TMAX + TPAD)];   // factored: R, R(d) at RPAD + d (padded layout)
  float z2[TMAX + TPAD];            // log2 Z
  float zi[padded(TMAX + TPAD)];          // factored: Zi (padded layout)
  float par[2 * TMAX];              // alpha, then rho (natural units)
  float mom[2 * TMAX], vel[2 * TMAX], tgt[2 * TMAX];   // Adam moments; col, then dist
  float rng[HW][4];                 // per wave: max alpha, -min alpha, max rho, -min rho
  double red[HW];
};

template <int TMAX>
__global__ __launch_bounds__(64 * HW) void fit_head_kernel(int T, int steps, AdamHyper hp,
                                                           const float* __restrict__ col,
                                                           const float* __restrict__ dist,
                                                           const float* __restrict__ ent,
                                                           float* __restrict__ alpha,
                                                           float* __restrict__ rho,
                                                           float* __restrict__ kl) {
  __shared__ __attribute__((aligned(16))) HeadFit<TMAX> sm;
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qd = lane >> 4, kl16 = lane & 15;
  const size_t hb = (size_t)h * T;
  const float inv_t = 1.f / T;

  // parameters, moments, targets; the padding of every table (entries [0, T) are written
  // at the start of each step)
  for (int x = tid; x < TMAX + TPAD; x += 64 * HW) {
    if (x < T) {
      sm.par[x] = alpha[hb + x];
      sm.par[T + x] = rho[hb + x];
      sm.tgt[x] = col[hb + x];
      sm.tgt[T + x] = dist[hb + x];
      sm.mom[x] = sm.mom[T + x] = 0.f;
      sm.vel[x] = sm.vel[T + x] = 0.f;
    } else {
      sm.a2[x] = 0.f;
      sm.r2[RPAD + x] = kNegInf;
      sm.fa[padx(x)] = 0.f;
      sm.fr[padx(RPAD + x)] = 0.f;
      sm.z2[x] = __builtin_huge_valf();
      sm.zi[padx(x)] = 0.f;
    }
  }
  if (tid < RPAD) {
    sm.r2[tid] = kNegInf;
    sm.fr[padx(tid)] = 0.f;
  }

  const int nb = (T + 15) / 16;   // 16-row (16-output) blocks
  // Block j of wave w: the waves take the blocks in rounds of HW, in reverse order every
  // other round, so that the lengths (which grow or shrink with the block index) even out.
  auto block_of = [&](int j) { return HW * j + ((j & 1) ? HW - 1 - w : w); };

  // log2 Z(i) of every row, exp path
  auto logz_exp = [&]() {
    for (int j = 0, u = block_of(0); u < nb; u = block_of(++j)) {
      const int i0 = 16 * u + 4 * qd;          // this lane group's rows i0 .. i0 + 3
      const int kend = min(16 * u + 15, T - 1);
      float mx[4] = {kNegInf, kNegInf, kNegInf, kNegInf}, s[4] = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 <= kend; k0 += 128) {
        const int k = k0 + 8 * kl16;           // keys k .. k + 7
        if (k > i0 + 3 || i0 >= T) continue;   // none of them in this lane's rows
        const float4 a0 = *reinterpret_cast<const float4*>(sm.a2 + k);
        const float4 a1 = *reinterpret_cast<const float4*>(sm.a2 + k + 4);
        // distances (i0 + q) - (k + e) = b + 8 + q - e with b = i0 - k - 8 >= -8, a multiple of 4
        const float* rb = sm.r2 + RPAD + (i0 - k - 8);
        const float4 w0 = *reinterpret_cast<const float4*>(rb);
        const float4 w1 = *reinterpret_cast<const float4*>(rb + 4);
        const float4 w2 = *reinterpret_cast<const float4*>(rb + 8);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float wv[12] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w2.x, w2.y, w2.z, w2.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float x[8];
          float cm = kNegInf;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = av[e] + wv[8 + q - e];
            cm = fmaxf(cm, x[e]);
          }
          // no branch for a row none of whose keys is here (cm = -inf): the reference is
          // then 0, so its exps are exp2(-inf) = 0 and the running sum keeps its value 0
          const float m_new = fmaxf(mx[q], cm);
          const float ref = m_new == kNegInf ? 0.f : m_new;
          float cs = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) cs += __builtin_amdgcn_exp2f(x[e] - ref);
          s[q] = s[q] * __builtin_amdgcn_exp2f(mx[q] - ref) + cs;
          mx[q] = m_new;
        }
      }
      float zr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float m = row16_max(mx[q]);
        const float t = row16_sum((mx[q] == kNegInf) ? 0.f : s[q] * __builtin_amdgcn_exp2f(mx[q] - m));
        zr[q] = m + __log2f(t);
      }
      if (kl16 < 4 && i0 + kl16 < T) sm.z2[i0 + kl16] = pick(zr, kl16);   // lane q: row i0 + q
    }
  };

  // log2 Z(i) and Zi(i) of every row, factored (32-row blocks, 8 rows per lane group);
  // top = max alpha2 + max rho2
  const int nb32 = (T + 31) / 32;
  auto logz_fac = [&](float top) {
    for (int j = 0, u = block_of(0); u < nb32; u = block_of(++j)) {
      const int i0 = 32 * u + 8 * qd;          // rows i0 .. i0 + 7
      const int kend = min(32 * u + 31, T - 1);
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 <= kend; k0 += 128) {
        const int k = k0 + 8 * kl16;
        if (k > i0 + 7 || i0 >= T) continue;
        const float4 a0 = *reinterpret_cast<const float4*>(sm.fa + padx(k));
        const float4 a1 = *reinterpret_cast<const float4*>(sm.fa + padx(k + 4));
        // distances (i0 + q) - (k + e) = b + 8 + q - e, b = i0 - k - 8 >= -8 (a multiple of 8)
        const int rb = RPAD + (i0 - k - 8);
        float wv[16];
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const float4 v = *reinterpret_cast<const float4*>(sm.fr + padx(rb + 4 * y));
          wv[4 * y] = v.x;
          wv[4 * y + 1] = v.y;
          wv[4 * y + 2] = v.z;
          wv[4 * y + 3] = v.w;
        }
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) s[q] = __builtin_fmaf(av[e], wv[8 + q - e], s[q]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] = row16_sum(s[q]);
      if (kl16 < 8 && i0 + kl16 < T) {   // lane q: row i0 + q
        const float t = pick(s, kl16);
        sm.z2[i0 + kl16] = top + __log2f(t);
        sm.zi[padx(i0 + kl16)] = 1.f / t;
      }
    }
  };

  // Adam on parameter k (alpha(x) at k = x, rho(d) at k = T + d) with marginal `sum`
  auto adam = [&](int k, float sum, float bc1, float bc2) {
    const float g = (sum - sm.tgt[k]) * inv_t;
    const float mm = hp.beta1 * sm.mom[k] + (1.f - hp.beta1) * g;
    const float vv = hp.beta2 * sm.vel[k] + (1.f - hp.beta2) * g * g;
    sm.mom[k] = mm;
    sm.vel[k] = vv;
    sm.par[k] = sm.par[k] - hp.lr * (mm / bc1) / (sqrtf(vv / bc2) + hp.eps);
  };

  // Marginals and the Adam step, exp path: output block u < nb: columns x = 16 u + 4 qd + c,
  // sum_t exp2(rho2(t) + alpha2(x) - z2(x + t)); u >= nb: distances (alpha and rho swapped).
  auto marginals_exp = [&](float bc1, float bc2) {
    for (int j = 0, u = block_of(0); u < 2 * nb; u = block_of(++j)) {
      const bool is_col = u < nb;
      const int x0 = 16 * (is_col ? u : u - nb) + 4 * qd;
      const float* own = is_col ? sm.a2 : sm.r2 + RPAD;
      const float* oth = is_col ? sm.r2 + RPAD : sm.a2;
      const int tend = T - 1 - 16 * (is_col ? u : u - nb);   // longest line of the block
      float ov[4], s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = own[x0 + c];
      for (int t0 = 0; t0 <= tend; t0 += 128) {
        const int t = t0 + 8 * kl16;           // terms t .. t + 7
        if (t > T - 1 - x0) continue;          // past the longest of this lane group's lines
        const float4 o0 = *reinterpret_cast<const float4*>(oth + t);
        const float4 o1 = *reinterpret_cast<const float4*>(oth + t + 4);
        const float* zb = sm.z2 + x0 + t;      // entry x0 + c + t + e is zb[c + e]
        const float4 z0 = *reinterpret_cast<const float4*>(zb);
        const float4 z1 = *reinterpret_cast<const float4*>(zb + 4);
        const float4 z3 = *reinterpret_cast<const float4*>(zb + 8);
        const float tv[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        const float zv[12] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w, z3.x, z3.y, z3.z, z3.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) s[c] += __builtin_amdgcn_exp2f(tv[e] + ov[c] - zv[c + e]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] = row16_sum(s[c]);
      const int x = x0 + kl16;   // lane c: output x0 + c
      if (kl16 < 4 && x < T) adam(is_col ? x : T + x, pick(s, kl16), bc1, bc2);
    }
  };

  // Marginals and the Adam step, factored: 32-output blocks, 8 outputs per lane group;
  // columns sum_t R(t) Zi(x + t) times A(x), distances sum_t A(t) Zi(d + t) times R(d).
  auto marginals_fac = [&](float bc1, float bc2) {
    for (int j = 0, u = block_of(0); u < 2 * nb32; u = block_of(++j)) {
      const bool is_col = u < nb32;
      const int x0 = 32 * (is_col ? u : u - nb32) + 8 * qd;
      // own(x) at padx(own_b + x), oth(t) at padx(oth_b + t)
      const float* own = is_col ? sm.fa : sm.fr;
      const float* oth = is_col ? sm.fr : sm.fa;
      const int own_b = is_col ? 0 : RPAD, oth_b = is_col ? RPAD : 0;
      const int tend = T - 1 - 32 * (is_col ? u : u - nb32);
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int t0 = 0; t0 <= tend; t0 += 128) {
        const int t = t0 + 8 * kl16;
        if (t > T - 1 - x0) continue;
        const float4 o0 = *reinterpret_cast<const float4*>(oth + padx(oth_b + t));
        const float4 o1 = *reinterpret_cast<const float4*>(oth + padx(oth_b + t + 4));
        float zv[16];   // Zi(x0 + t + y), y = c + e
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const float4 v = *reinterpret_cast<const float4*>(sm.zi + padx(x0 + t + 4 * y));
          zv[4 * y] = v.x;
          zv[4 * y + 1] = v.y;
          zv[4 * y + 2] = v.z;
          zv[4 * y + 3] = v.w;
        }
        const float tv[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) s[c] = __builtin_fmaf(tv[e], zv[c + e], s[c]);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) s[c] = row16_sum(s[c]);
      const int x = x0 + kl16;   // lane c: output x0 + c
      if (kl16 < 8 && x < T) adam(is_col ? x : T + x, pick(s, kl16) * own[padx(own_b + x)], bc1, bc2);
    }
  };

  double p1 = 1.0, p2 = 1.0;
  for (int step = 1;; ++step) {
    // spreads of the current parameters (all waves end up with the same values)
    float st[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
    for (int x = tid; x < T; x += 64 * HW) {
      const float a = sm.par[x], r = sm.par[T + x];
      st[0] = fmaxf(st[0], a);
      st[1] = fmaxf(st[1], -a);
      st[2] = fmaxf(st[2], r);
      st[3] = fmaxf(st[3], -r);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      st[c] = wave_max(st[c]);
      if (lane == 0) sm.rng[w][c] = st[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      st[c] = sm.rng[0][c];
      for (int v = 1; v < HW; ++v) st[c] = fmaxf(st[c], sm.rng[v][c]);
    }
    const float am2 = st[0] * kLog2e, rm2 = st[2] * kLog2e;
    // false for a NaN or infinite spread
    const bool fac = (st[0] + st[1] + st[2] + st[3]) * kLog2e <= kFactorSpread;
    for (int x = tid; x < T; x += 64 * HW) {
      const float a = sm.par[x] * kLog2e, r = sm.par[T + x] * kLog2e;
      if (fac) {
        sm.fa[padx(x)] = __builtin_amdgcn_exp2f(a - am2);
        sm.fr[padx(RPAD + x)] = __builtin_amdgcn_exp2f(r - rm2);
      } else {
        sm.a2[x] = a;
        sm.r2[RPAD + x] = r;
      }
    }
    __syncthreads();
    if (fac) logz_fac(am2 + rm2);
    else logz_exp();
    __syncthreads();
    if (step > steps) break;
    p1 *= hp.beta1;
    p2 *= hp.beta2;
    if (fac) marginals_fac((float)(1.0 - p1), (float)(1.0 - p2));
    else marginals_exp((float)(1.0 - p1), (float)(1.0 - p2));
    __syncthreads();
  }

  // the fitted tables, and the mean row KL (1/T) [sum log Z - alpha.col - rho.dist - sum ent]
  double acc = 0.0;
  for (int x = tid; x < T; x += 64 * HW) {
    const float a = sm.par[x], r = sm.par[T + x];
    alpha[hb + x] = a;
    rho[hb + x] = r;
    acc += (double)(sm.z2[x] * kLn2) - (double)a * sm.tgt[x] - (double)r * sm.tgt[T + x] - (double)ent[hb + x];
  }
  acc = wave_sum(acc);
  if (lane == 0) sm.red[w] = acc;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int x = 0; x < HW; ++x) t += sm.red[x];
    kl[h] = (float)(t / T);
  }
}

int elementwise_blocks(size_t n) { return (int)std::min<size_t>((n + 255) / 256, 4096); }

size_t pad64(size_t n) { return (n + 63) / 64 * 64; }

}  // namespace

hipError_t launch_pattern_stats(int H, int T, const float* a, float* col, float* dist, float* ent,
                                hipStream_t s) {
  prof_begin("fit_stats", s);
  hipLaunchKernelGGL(stats_kernel, dim3((T + 63) / 64, H), dim3(64 * SW), 0, s, T, a, col, dist, ent);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_compact_marginals(int H, int T, const float* alpha, const float* rho, float* logz,
                                    float* col_p, float* dist_p, hipStream_t s) {
  const int nb = (T + OPW * LW - 1) / (OPW * LW);
  prof_begin("fit_logz", s);
  hipLaunchKernelGGL(logz_kernel, dim3(nb, H), dim3(64 * LW), 0, s, T, alpha, rho, logz);
  prof_end(s);
  prof_begin("fit_marginals", s);
  hipLaunchKernelGGL(marg_kernel<false>, dim3(2 * nb, H), dim3(64 * LW), 0, s, T, nb, alpha,
                     rho, (const float*)logz, col_p, dist_p, (const float*)nullptr, (const float*)nullptr,
                     (float*)nullptr, (float*)nullptr, AdamStep{});
  prof_end(s);
  return hipGetLastError();
}

size_t fit_workspace_floats(int H, int T) { return 7 * pad64((size_t)H * T); }

bool fit_per_head(const FitArgs& f) {
  if (f.schedule == kFitPerHead) return true;
  return f.schedule == kFitAuto && f.T <= kFitHeadMaxT && (f.H >= kFitHeadMinHeads || f.T <= kFitHeadShortT);
}

hipError_t launch_compact_fit(const FitArgs& f, const float* col, const float* dist, const float* ent,
                              float* alpha, float* rho, float* kl, float* ws, hipStream_t s) {
  const int H = f.H, T = f.T;
  if (fit_per_head(f)) {
    const AdamHyper hp{f.lr, f.beta1, f.beta2, f.eps};
    prof_begin("fit_head", s);
    if (T <= 1024)
      hipLaunchKernelGGL(fit_head_kernel<1024>, dim3(H), dim3(64 * HW), 0, s, T, f.steps, hp, col, dist, ent,
                         alpha, rho, kl);
    else
      hipLaunchKernelGGL(fit_head_kernel<kFitHeadMaxT>, dim3(H), dim3(64 * HW), 0, s, T, f.steps, hp, col, dist,
                         ent, alpha, rho, kl);
    prof_end(s);
    return hipGetLastError();
  }
  const size_t n = pad64((size_t)H * T);
  float* logz = ws;
  float* alt_alpha = ws + n;
  float* alt_rho = ws + 2 * n;
  float* m = ws + 3 * n;       // [H, 2T]
  float* v = ws + 5 * n;       // [H, 2T]
  hipLaunchKernelGGL(fill_kernel, dim3(elementwise_blocks(4 * n)), dim3(256), 0, s, m, 4 * n, 0.f);
  float* cur[2] = {alpha, rho};
  float* nxt[2] = {alt_alpha, alt_rho};
  const int nb = (T + OPW * LW - 1) / (OPW * LW);
  const dim3 lz_grid(nb, H), mg_grid(2 * nb, H), blk(64 * LW);
  double p1 = 1.0, p2 = 1.0;
  for (int t = 1; t <= f.steps; ++t) {
    p1 *= f.beta1;
    p2 *= f.beta2;
    const AdamStep st{f.lr, f.beta1, f.beta2, f.eps, (float)(1.0 - p1), (float)(1.0 - p2), 1.f / T};
    prof_begin("fit_logz", s);
    hipLaunchKernelGGL(logz_kernel, lz_grid, blk, 0, s, T, (const float*)cur[0], (const float*)cur[1], logz);
    prof_end(s);
    prof_begin("fit_adam", s);
    hipLaunchKernelGGL(marg_kernel<true>, mg_grid, blk, 0, s, T, nb, (const float*)cur[0], (const float*)cur[1],
                       (const float*)logz, nxt[0], nxt[1], col, dist, m, v, st);
    prof_end(s);
    std::swap(cur[0], nxt[0]);
    std::swap(cur[1], nxt[1]);
  }
  if (cur[0] != alpha) {
    hipLaunchKernelGGL(copy_kernel, dim3(elementwise_blocks((size_t)H * T)), dim3(256), 0, s, alpha,
                       (const float*)cur[0], (size_t)H * T);
    hipLaunchKernelGGL(copy_kernel, dim3(elementwise_blocks((size_t)H * T)), dim3(256), 0, s, rho,
                       (const float*)cur[1], (size_t)H * T);
  }
  hipLaunchKernelGGL(logz_kernel, lz_grid, blk, 0, s, T, (const float*)alpha, (const float*)rho, logz);
  hipLaunchKernelGGL(kl_kernel, dim3(H), dim3(256), 0, s, T, (const float*)alpha, (const float*)rho,
                     (const float*)logz, col, dist, ent, kl);
  return hipGetLastError();
}

}  // namespace saf
