// Hybrid causal attention forward, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// Method: "When Can Attention Heads Be Statically Defined?: 中文精读笔记".
//   ordinary head (part 一):  O = softmax_causal(scale Q K^T) V
//   frozen head (part 二.3, Eq. (3); part 二.4, Fig. 2):
//       O(i) = sum_{j<=i} exp(alpha(j) + rho(i-j) - log Z(i)) V(j)
// The page's fused kernel rebuilds a frozen tile from alpha, rho and Z and multiplies it
// by V, with ordinary heads on flash-style online-softmax tiles, in one launch per layer.
// Here both kinds of work items share one launch as well; the tiling is our own, built
// around 64-wide wavefronts and the 32x32x16 bf16 MFMA.
//
// Work items (one 256-thread workgroup each, 4 waves x 32 queries = a 128-query tile):
//   dynamic (b, h, q-tile): S^T = K Q^T per 64-key tile (each lane keeps one query),
//       online softmax in log2 units with a lazy rescale (the running max is only raised
//       when a tile exceeds it by more than 2^8), O^T += V^T P^T;
//   frozen (h, q-tile, column chunk): the batch is folded into the columns, so one
//       item multiplies the regenerated pattern tile by up to 256 columns of
//       [V_0 | V_1 | ...] and the exp work is shared by every batch entry.
// Items are issued heaviest q-tile first; key tiles above the causal diagonal are skipped.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

constexpr int BM = 128;        // queries per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int NTH = 256;
constexpr int FCOLS = 256;     // batch-folded columns per frozen item
constexpr float kRescaleSlack = 8.0f;  // log2 units

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* alpha;
  const float* rho;
  bf16* o;
  float* lse;
  int tab_stride;
  int B, H, T;
  float c;  // scale * log2(e)
  int n_dyn, n_frz, n_qt, n_chunks, per_qt;
  uint8_t dyn[kMaxHeads];
  uint8_t frz[kMaxHeads];
};

template <int D>
struct DynSmem {
  bf16 k[BN * D];   // row-major key tile, 16-byte chunks swizzled by swz_pi(row)
  bf16 vt[D * BN];  // transposed value tile [d][key], chunks swizzled by swz_tr(d)
};

struct FrzSmem {
  bf16 vt[FCOLS * BN];   // transposed folded value tile [column][key]
  float a2[BN];          // alpha * log2(e) of the tile's keys
  float rw[BM + BN];     // rho * log2(e) over the tile's distance window
};

template <int D>
constexpr int smem_bytes() {
  return sizeof(DynSmem<D>) > sizeof(FrzSmem) ? (int)sizeof(DynSmem<D>) : (int)sizeof(FrzSmem);
}

// ---------------------------------------------------------------- dynamic item

template <int D>
__device__ void dyn_item(const FwdParams& p, int b, int h, int qt, unsigned char* smem_raw) {
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int NKC = BN * CPR / NTH;     // key-tile chunks per thread
  constexpr int NVB = (BN / 4) * CPR;     // 4x8 value blocks per tile
  DynSmem<D>& sm = *reinterpret_cast<DynSmem<D>*>(smem_raw);
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const int m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const size_t head = ((size_t)b * p.H + h) * (size_t)T;
  const bf16* Q = p.q + head * D;
  const bf16* K = p.k + head * D;
  const bf16* V = p.v + head * D;
  const int i0w = qt * BM + w * 32;
  const int i = i0w + m;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (i < T) qf[kk] = *reinterpret_cast<const bf16x8*>(Q + (size_t)i * D + kk * 16 + hh * 8);
    else qf[kk] = bf16x8{};
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_used = kNegInf, l = 0.f;

  const int n_kt = min(2 * qt + 2, (T + BN - 1) / BN);

  u32x4 kreg[NKC];
  u32x4 vreg[4];
  auto gload = [&](int J) {
    const int j0 = J * BN;
#pragma unroll
    for (int x = 0; x < NKC; ++x) {
      const int c = t + NTH * x, row = c / CPR, cc = c % CPR;
      kreg[x] = (j0 + row < T) ? *reinterpret_cast<const u32x4*>(K + (size_t)(j0 + row) * D + cc * 8)
                               : u32x4{0, 0, 0, 0};
    }
    if (t < NVB) {
      const int db = t % CPR, kg = t / CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + 4 * kg + r;
        vreg[r] = (key < T) ? *reinterpret_cast<const u32x4*>(V + (size_t)key * D + db * 8)
                            : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int x = 0; x < NKC; ++x) {
      const int c = t + NTH * x, row = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(sm.k + row * D + ((cc ^ swz_pi(row)) * 8)) = kreg[x];
    }
    if (t < NVB) {
      const int db = t % CPR, kg = t / CPR;
      u32x2 cols[8];
      transpose_4x8(vreg, cols);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int d = db * 8 + c;
        *reinterpret_cast<u32x2*>(sm.vt + d * BN + (((kg >> 1) ^ swz_tr(d)) * 8) + (kg & 1) * 4) = cols[c];
      }
    }
  };

  gload(0);
  sstore();
  __syncthreads();
  for (int J = 0; J < n_kt; ++J) {
    if (J + 1 < n_kt) gload(J + 1);
    const int j0 = J * BN;
    if (j0 <= i0w) {  // tile meets this wave's causal region
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int krow = kb * 32 + perm_rows(m);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const int ch = 2 * kk + hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.k + krow * D + ((ch ^ swz_pi(krow)) * 8));
          s[kb] = mfma32(a, qf[kk], s[kb]);
        }
      }
      if (j0 + BN - 1 > i0w) {  // diagonal tile: mask keys after the query
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (j0 + kb * 32 + acc_pos(r, hh) > i) s[kb][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, wave_shfl_xor32(mx));
      const float mt = mx * p.c;
      const bool up = mt > m_used + kRescaleSlack;
      if (__any(up)) {
        const float m_new = up ? mt : m_used;
        const float alpha = (m_used == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_used - m_new);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        l *= alpha;
        m_used = m_new;
      }
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], p.c, -m_used));
          l += pv[r];
        }
        pb[2 * kb] = pack8(pv);
        pb[2 * kb + 1] = pack8(pv + 8);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + m;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int ch = 2 * ks + hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.vt + d * BN + ((ch ^ swz_tr(d)) * 8));
          o[db] = mfma32(a, pb[ks], o[db]);
        }
      }
    }
    __syncthreads();
    if (J + 1 < n_kt) {
      sstore();
      __syncthreads();
    }
  }

  const float lt = l + wave_shfl_xor32(l);
  if (i < T) {
    const float inv = 1.f / lt;
    bf16* O = p.o + head * D + (size_t)i * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + acc_row(4 * g, hh);
        u32x2 pk;
        pk[0] = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        pk[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(O + d) = pk;
      }
    if (hh == 0) p.lse[head + i] = (m_used + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------- frozen item

template <int D>
__device__ void frz_item(const FwdParams& p, int h, int chunk, int qt, unsigned char* smem_raw) {
  FrzSmem& sm = *reinterpret_cast<FrzSmem*>(smem_raw);
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const int m = lane & 31, hh = lane >> 5;
  const int T = p.T, H = p.H;
  const int ncol_all = p.B * D;
  const int col0 = chunk * FCOLS;
  const int ncols = min(FCOLS, ncol_all - col0);
  const int i0 = qt * BM, i0w = i0 + w * 32, i = i0w + m;
  const float* alpha = p.alpha + (size_t)h * p.tab_stride;
  const float* rho = p.rho + (size_t)h * p.tab_stride;
  const float lz = (i < T) ? p.lse[(size_t)h * T + i] * kLog2e : 0.f;  // log Z(i), batch 0

  f32x16 o[FCOLS / 32];
#pragma unroll
  for (int cb = 0; cb < FCOLS / 32; ++cb) o[cb] = f32x16{};

  const int n_kt = min(2 * qt + 2, (T + BN - 1) / BN);
  constexpr int NVB = (BN / 4) * (FCOLS / 8);  // 4x8 blocks per tile = 512
  u32x4 vreg[NVB / NTH][4];
  float treg;
  auto gload = [&](int J) {
    const int j0 = J * BN;
#pragma unroll
    for (int x = 0; x < NVB / NTH; ++x) {
      const int blk = t + NTH * x, cg = blk % (FCOLS / 8), kg = blk / (FCOLS / 8);
      const int col = col0 + cg * 8;
      const bool ok = cg * 8 < ncols;
      const int bb = col / D, d = col % D;
      const bf16* Vb = p.v + (((size_t)bb * H + h) * T) * D + d;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + 4 * kg + r;
        vreg[x][r] = (ok && key < T) ? *reinterpret_cast<const u32x4*>(Vb + (size_t)key * D)
                                     : u32x4{0, 0, 0, 0};
      }
    }
    if (t < BN) {
      treg = (j0 + t < T) ? alpha[j0 + t] * kLog2e : kNegInf;
    } else if (t < BN + BM + BN - 1) {
      const int dd = i0 - j0 - (BN - 1) + (t - BN);
      treg = (dd >= 0 && dd < T) ? rho[dd] * kLog2e : kNegInf;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int x = 0; x < NVB / NTH; ++x) {
      const int blk = t + NTH * x, cg = blk % (FCOLS / 8), kg = blk / (FCOLS / 8);
      u32x2 cols[8];
      transpose_4x8(vreg[x], cols);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = cg * 8 + c;
        *reinterpret_cast<u32x2*>(sm.vt + col * BN + (((kg >> 1) ^ swz_tr(col)) * 8) + (kg & 1) * 4) = cols[c];
      }
    }
    if (t < BN) sm.a2[t] = treg;
    else if (t < BN + BM + BN - 1) sm.rw[t - BN] = treg;
  };

  gload(0);
  sstore();
  __syncthreads();
  for (int J = 0; J < n_kt; ++J) {
    if (J + 1 < n_kt) gload(J + 1);
    const int j0 = J * BN;
    if (j0 <= i0w) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float pv[8];
        const int kofs = ks * 16 + hh * 8;
        // distance window index of (i, j0 + kofs + e) is (i - i0) - (kofs + e) + BN - 1;
        // entries for j > i hold -inf, so the causal mask comes for free.
        const int rbase = (i - i0) - kofs + BN - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pv[e] = __builtin_amdgcn_exp2f(sm.a2[kofs + e] + sm.rw[rbase - e] - lz);
        const bf16x8 pb = pack8(pv);
#pragma unroll
        for (int cb = 0; cb < FCOLS / 32; ++cb) {
          if (cb * 32 < ncols) {
            const int col = cb * 32 + m;
            const int ch = 2 * ks + hh;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.vt + col * BN + ((ch ^ swz_tr(col)) * 8));
            o[cb] = mfma32(a, pb, o[cb]);
          }
        }
      }
    }
    __syncthreads();
    if (J + 1 < n_kt) {
      sstore();
      __syncthreads();
    }
  }

  if (i < T) {
#pragma unroll
    for (int cb = 0; cb < FCOLS / 32; ++cb) {
      if (cb * 32 >= ncols) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + cb * 32 + acc_row(4 * g, hh);
        const int bb = col / D, d = col % D;
        u32x2 pk;
        pk[0] = pack_bf16x2(o[cb][4 * g], o[cb][4 * g + 1]);
        pk[1] = pack_bf16x2(o[cb][4 * g + 2], o[cb][4 * g + 3]);
        *reinterpret_cast<u32x2*>(p.o + (((size_t)bb * H + h) * T + i) * D + d) = pk;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(NTH, 2) void hybrid_fwd_kernel(const FwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[smem_bytes<D>()];
  const int item = blockIdx.x;
  const int qt = p.n_qt - 1 - item / p.per_qt;
  int rem = item % p.per_qt;
  const int nd = p.B * p.n_dyn;
  if (rem < nd) {
    dyn_item<D>(p, rem / p.n_dyn, p.dyn[rem % p.n_dyn], qt, smem);
  } else {
    rem -= nd;
    frz_item<D>(p, p.frz[rem / p.n_chunks], rem % p.n_chunks, qt, smem);
  }
}

// ---------------------------------------------------------------- log Z prologue

struct LogzParams {
  const float* alpha;
  const float* rho;
  float* lse;
  int tab_stride, B, H, T;
  uint8_t frz[kMaxHeads];
};

// log Z(i) = log sum_{j<=i} exp(alpha(j) + rho(i-j)) (Eq. (3)), max-subtracted, one row per
// 8 lanes; written to lse[b, h, i] for every b. Batch independent.
__global__ __launch_bounds__(256) void frozen_logz_kernel(const LogzParams p) {
  const int h = p.frz[blockIdx.y];
  const int row = blockIdx.x * 32 + (threadIdx.x >> 3), sub = threadIdx.x & 7;
  const float* al = p.alpha + (size_t)h * p.tab_stride;
  const float* rh = p.rho + (size_t)h * p.tab_stride;
  float mx = kNegInf;
  if (row < p.T)
    for (int j = sub; j <= row; j += 8) mx = fmaxf(mx, al[j] + rh[row - j]);
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float s = 0.f;
  if (row < p.T)
    for (int j = sub; j <= row; j += 8) s += exp2f((al[j] + rh[row - j] - mx) * kLog2e);
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) s += __shfl_xor(s, o, 64);
  if (row < p.T && sub == 0) {
    const float lz = mx + logf(s);
    for (int b = 0; b < p.B; ++b) p.lse[((size_t)b * p.H + h) * p.T + row] = lz;
  }
}

}  // namespace

hipError_t launch_frozen_logz(const AttnArgs& a, const float* alpha, const float* rho,
                              float* lse, hipStream_t s) {
  if (a.heads.n_frz == 0) return hipSuccess;
  LogzParams p;
  p.alpha = alpha;
  p.rho = rho;
  p.lse = lse;
  p.tab_stride = a.tab_stride;
  p.B = a.B;
  p.H = a.H;
  p.T = a.T;
  for (int x = 0; x < kMaxHeads; ++x) p.frz[x] = a.heads.frz[x];
  dim3 grid((a.T + 31) / 32, a.heads.n_frz);
  prof_begin("frozen_logz", s);
  hipLaunchKernelGGL(frozen_logz_kernel, grid, dim3(256), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const float* alpha, const float* rho, void* o, float* lse,
                           hipStream_t s) {
  FwdParams p;
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.alpha = alpha;
  p.rho = rho;
  p.o = static_cast<bf16*>(o);
  p.lse = lse;
  p.tab_stride = a.tab_stride;
  p.B = a.B;
  p.H = a.H;
  p.T = a.T;
  p.c = a.scale * kLog2e;
  p.n_dyn = a.heads.n_dyn;
  p.n_frz = a.heads.n_frz;
  p.n_qt = (a.T + BM - 1) / BM;
  p.n_chunks = (a.B * a.D + FCOLS - 1) / FCOLS;
  p.per_qt = a.B * p.n_dyn + p.n_frz * p.n_chunks;
  for (int x = 0; x < kMaxHeads; ++x) {
    p.dyn[x] = a.heads.dyn[x];
    p.frz[x] = a.heads.frz[x];
  }
  const int n_items = p.n_qt * p.per_qt;
  if (n_items == 0) return hipSuccess;
  prof_begin("hybrid_fwd", s);
  if (a.D == 64)
    hipLaunchKernelGGL(hybrid_fwd_kernel<64>, dim3(n_items), dim3(NTH), 0, s, p);
  else
    hipLaunchKernelGGL(hybrid_fwd_kernel<128>, dim3(n_items), dim3(NTH), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
