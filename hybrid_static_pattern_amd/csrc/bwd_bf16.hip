// Hybrid causal attention backward, bf16 inputs, fp32 gradients, gfx950 MFMA.
//
// Method: "When Can Attention Heads Be Statically Defined?: 中文精读笔记".
//   ordinary heads: the textbook softmax-attention gradient of part 一's layer,
//       dV = A^T dO, dS = A o (dO V^T - delta), dQ = scale dS K, dK = scale dS^T Q,
//       delta_i = sum_c dO_ic O_ic, with A recomputed from the saved log-normaliser;
//   frozen heads (part 二.4 / Algorithm 1): alpha and rho are fixed buffers without
//       gradient and there is no query or key, so the only gradient is dV = P^T dO,
//       P rebuilt from alpha, rho and log Z exactly as in the forward (Eq. (3)).
//
// Kernels, in launch order:
//   bwd_delta   delta for ordinary heads (one 8-lane group per row);
//   dkdv        one launch of 8-wave workgroups on 16x16x32 MFMAs, two kinds of items:
//       ordinary (b, h, 128-key tile): each wave keeps 16 keys (K, V fragments and the
//           fp32 dK, dV tiles) in registers and walks the 64-query steps from the
//           diagonal down; S and dP are computed with the key as the lane index so P
//           and dS feed the dV and dK products straight from registers;
//       frozen (h, 128-key tile, column chunk): the batch is folded into up to 256
//           columns of [dO_0 | dO_1 | ...]; P^T is regenerated per lane and split into a
//           bf16 high and low part (two MFMAs) so the fp32 dV keeps ~16 bits of P;
//   dq          ordinary (b, h, 128-query tile), keys from 0 to the diagonal, the query
//           as the lane index (as in the forward): dQ = scale * sum_J dS K_J.
// Q/dO (dK/dV kernel) and K/V (dQ kernel) tiles go from HBM straight into double-buffered
// LDS, one barrier per step; the transposed operands (dO^T, Q^T, K^T) are read from the
// same row-major tiles with ds_read_b64_tr_b16. The split into a key-stationary and a query-stationary kernel recomputes S and dP once
// more instead of accumulating dQ with atomics; every output is written exactly once.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

constexpr int NTH = 256;
constexpr int BNK = 128;   // keys per dK/dV workgroup
constexpr int BMQ = 64;    // queries per dK/dV step
constexpr int BMD = 128;   // queries per dQ workgroup
constexpr int BND = 64;    // keys per dQ step
constexpr int FCOLS = 256;

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dO;
  const float* lse;
  const float* delta;
  const float* alpha;
  const float* rho;
  float* dq;
  float* dk;
  float* dv;
  int tab_stride, B, H, T;
  float c;      // scale * log2(e)
  float scale;
  int n_dyn, n_frz, n_chunks, per_tile, n_tiles;
  uint8_t dyn[kMaxHeads];
  uint8_t frz[kMaxHeads];
};

// ---------------------------------------------------------------- delta

struct DeltaParams {
  const void* o;
  const void* dO;
  float* delta;
  int H, T, D, n_rows;  // n_rows = B * n_dyn * T
  int n_dyn;
  bool bf16;
  uint8_t dyn[kMaxHeads];
};

__global__ __launch_bounds__(256) void bwd_delta_kernel(const DeltaParams p) {
  const int row = blockIdx.x * 32 + (threadIdx.x >> 3), sub = threadIdx.x & 7;
  float acc = 0.f;
  size_t r = 0;
  if (row < p.n_rows) {
    const int i = row % p.T, bh = row / p.T;
    const int h = p.dyn[bh % p.n_dyn], b = bh / p.n_dyn;
    r = ((size_t)b * p.H + h) * p.T + i;
    if (p.bf16) {
      const uint16_t* O = static_cast<const uint16_t*>(p.o) + r * p.D;
      const uint16_t* G = static_cast<const uint16_t*>(p.dO) + r * p.D;
      for (int d = sub * 8; d < p.D; d += 64) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(O + d);
        const u32x4 g = *reinterpret_cast<const u32x4*>(G + d);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          acc = fmaf(bf16_to_f32(a[x] & 0xffff), bf16_to_f32(g[x] & 0xffff), acc);
          acc = fmaf(bf16_to_f32(a[x] >> 16), bf16_to_f32(g[x] >> 16), acc);
        }
      }
    } else {
      const float* O = static_cast<const float*>(p.o) + r * p.D;
      const float* G = static_cast<const float*>(p.dO) + r * p.D;
      for (int d = sub * 4; d < p.D; d += 32) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(O + d);
        const f32x4 g = *reinterpret_cast<const f32x4*>(G + d);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc = fmaf(a[x], g[x], acc);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (row < p.n_rows && sub == 0) p.delta[r] = acc;
}

// ---------------------------------------------------------------- dK / dV

// ---------------------------------------------------------------- dK / dV, ordinary heads
//
// 8 waves x 16 keys per 128-key workgroup on v_mfma_f32_16x16x32_bf16, so that a wave's
// fp32 dK and dV tiles (16 keys x D) take 64 registers and two waves fit on each SIMD: while
// one wave runs its softmax arithmetic the other keeps the matrix cores busy.
//   16x16x32 operand layout: A (16 x 32): lane l holds A[l % 16][8 (l / 16) + e];
//   B (32 x 16): lane l holds B[8 (l / 16) + e][l % 16]; C (16 x 16): lane l, register r
//   holds C[4 (l / 16) + r][l % 16].
// S = Q K^T is computed in two 16-query halves h whose A rows are the step's Q rows
// 8 (rho / 4) + 4 h + rho % 4 (rho = MFMA row): then register r of half h in lane group g
// holds query 8 g + 4 h + r, and the 8 values of lane group g are exactly the 8 consecutive
// queries 8 g .. 8 g + 7 that the P^T operand of the dV product needs (k index e = 4 h + r).

constexpr int NW16 = 8;            // waves per ordinary dK/dV workgroup
constexpr int NTH16 = 64 * NW16;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Chunk swizzle for the 16-lane read patterns of this kernel (period 32 in the row):
//   A rows: each 16-lane group reads rows {0..3, 8..11, 16..19, 24..27} (+4, +32) at one chunk;
//   B via ds_read_b64_tr_b16: each half-wave reads rows {0..3, 8..11} (+16, +4, +32) over
//   32 bytes. Both map to distinct banks with 64 four-byte banks.
template <int CPR>
__device__ __forceinline__ int swz16(int r) {
  return CPR >= 16 ? (((r & 3) << 1) | (((r >> 3) & 1) << 3) | ((r >> 4) & 1))
                   : (((r >> 4) & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2));
}

template <int CPR, int NR, class Src>
__device__ __forceinline__ void tile_load16(bf16* tile, Src src) {
  constexpr int NCH = NR * CPR;
  constexpr int PERW = NCH / 64 / NW16;
  static_assert(NCH % (64 * NW16) == 0, "tile must split evenly over the waves");
  const int w = wave_id(), lane = lane_id();
  const uint32_t base = lds_addr(tile);
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int blk = w * PERW + x;
    const int pch = blk * 64 + lane;
    const int row = pch / CPR;
    const int c = (pch % CPR) ^ swz16<CPR>(row);
    g2lds16(src(row, c), base + blk * 1024);
  }
}

template <int D>
struct Dkdv16Stage {
  bf16 qs[BMQ * D];   // Q rows of the step, swizzled (swz16)
  bf16 gs[BMQ * D];   // dO rows of the step
  float ls[BMQ];      // lse * log2(e) (+inf past T)
  float dl[BMQ];      // delta
};

struct Frz16Stage {
  bf16 gs[BMQ * FCOLS];   // folded dO [q][column], swizzled (swz16); read transposed
  float lz[BMQ];          // log Z * log2(e) (+inf past T)
  float rw[BMQ + BNK];    // rho * log2(e) over the step's distance window
};

template <int D>
constexpr int dkdv16_smem_bytes() {
  return 2 * (sizeof(Dkdv16Stage<D>) > sizeof(Frz16Stage) ? (int)sizeof(Dkdv16Stage<D>) : (int)sizeof(Frz16Stage));
}

// Frozen item (h, 128-key tile, column chunk): dV_b[j] = sum_{i>=j} P(i,j) dO_b[i] for the
// batch folded into up to 256 columns. Each wave keeps 16 keys x 256 columns of fp32 dV;
// P^T is regenerated per lane from alpha, rho and log Z (entries for j > i come out as 0 from
// the -inf distances of the window) and split into bf16 high and low parts.
template <int D>
__device__ void dv_frz16(const BwdParams& p, int h, int chunk, int kt, unsigned char* smem_raw) {
  constexpr int CPR = FCOLS / 8;
  constexpr int NCB = FCOLS / 16;
  Frz16Stage* stg = reinterpret_cast<Frz16Stage*>(smem_raw);
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int T = p.T, H = p.H, B = p.B;
  const int col0 = chunk * FCOLS;
  const int ncols = min(FCOLS, B * D - col0);
  const int kbase = kt * BNK, k0w = kbase + 16 * w, j = k0w + n;
  const float a2 = (j < T) ? p.alpha[(size_t)h * p.tab_stride + j] * kLog2e : kNegInf;
  const float* rho = p.rho + (size_t)h * p.tab_stride;

  f32x4 dv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dv[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t goff[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 8 * g + ((lane >> 2) & 3) + 4 * hf, col = 16 * cb + 4 * (lane & 3);
      goff[cb][hf] = 2u * (uint32_t)(row * FCOLS + (((col >> 3) ^ swz16<CPR>(row)) << 3) + (col & 7));
    }

  const int n_steps = (T - kbase + BMQ - 1) / BMQ;
  constexpr int NTAB = BMQ + BMQ + BNK - 1;   // lz for the step's queries, then the rho window
  static_assert(NTAB <= NTH16, "one table entry per thread");
  float treg = 0.f;
  auto load = [&](int st, Frz16Stage& sm) {
    const int i0 = kbase + st * BMQ;
    tile_load16<CPR, BMQ>(sm.gs, [&](int row, int c) {
      const int col = col0 + c * 8;
      const int bb = min(col / D, B - 1), d = col % D;
      return p.dO + (((size_t)bb * H + h) * T + min(i0 + row, T - 1)) * D + d;
    });
    if (t < BMQ) {
      const int i = i0 + t;
      treg = (i < T) ? p.lse[(size_t)h * T + i] * kLog2e : __builtin_huge_valf();
    } else if (t < NTAB) {
      const int dd = i0 - kbase - (BNK - 1) + (t - BMQ);
      treg = (dd >= 0 && dd < T) ? rho[dd] * kLog2e : kNegInf;
    }
  };
  auto store_tables = [&](Frz16Stage& sm) {
    if (t < BMQ) sm.lz[t] = treg;
    else if (t < NTAB) sm.rw[t - BMQ] = treg;
  };

  auto step = [&](int st, const Frz16Stage& sm, Frz16Stage& nxt) {
    if (st + 1 < n_steps) load(st + 1, nxt);
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) {
      if (st * (BMQ / 32) + qb < (w >> 1)) continue;   // every query before this wave's keys
      // queries i0 + qb*32 + 8 g + e; window index of distance i - j is
      // (qb*32 + 8 g + e) - (16 w + n) + BNK - 1
      const int qofs = qb * 32 + 8 * g;
      const int rbase = qofs - (16 * w + n) + BNK - 1;
      float ph[8], pl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = __builtin_amdgcn_exp2f(a2 + sm.rw[rbase + e] - sm.lz[qofs + e]);
        const bf16 hi = (bf16)pv;
        ph[e] = (float)hi;
        pl[e] = pv - ph[e];
      }
      const bf16x8 ahi = pack8(ph), alo = pack8(pl);
      pipelined<NCB>(
          [&](int cb) {
            const char* base = reinterpret_cast<const char*>(sm.gs) + qb * 32 * (CPR * 16);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + goff[cb][0]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + goff[cb][1]));
            u32x4 r;
            r[0] = __builtin_bit_cast(u32x2, lo)[0];
            r[1] = __builtin_bit_cast(u32x2, lo)[1];
            r[2] = __builtin_bit_cast(u32x2, hi)[0];
            r[3] = __builtin_bit_cast(u32x2, hi)[1];
            return __builtin_bit_cast(bf16x8, r);
          },
          [&](int cb, const bf16x8& bg) {
            dv[cb] = mfma16(ahi, bg, dv[cb]);
            dv[cb] = mfma16(alo, bg, dv[cb]);
          });
    }
    if (st + 1 < n_steps) store_tables(nxt);
    wait_vm0();
    __syncthreads();
  };

  load(0, stg[0]);
  store_tables(stg[0]);
  wait_vm0();
  __syncthreads();
  for (int st = 0; st < n_steps; st += 2) {  // unrolled by two: the LDS stage is a constant
    step(st, stg[0], stg[1]);
    if (st + 1 < n_steps) step(st + 1, stg[1], stg[0]);
  }

#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int col = col0 + 16 * cb + n;
    if (16 * cb >= ncols) continue;
    const int bb = col / D, d = col % D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0w + 4 * g + r;
      if (key < T) p.dv[(((size_t)bb * H + h) * T + key) * D + d] = dv[cb][r];
    }
  }
}

template <int D>
__device__ void dkdv_dyn16(const BwdParams& p, int b, int h, int kt, unsigned char* smem_raw) {
  constexpr int CPR = D / 8;
  constexpr int NKS = D / 32;   // 32-wide k-steps over d
  constexpr int NDB = D / 16;   // 16-wide d blocks of dK, dV
  Dkdv16Stage<D>* stg = reinterpret_cast<Dkdv16Stage<D>*>(smem_raw);
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int T = p.T;
  const size_t head = ((size_t)b * p.H + h) * (size_t)T;
  const bf16* Q = p.q + head * D;
  const bf16* G = p.dO + head * D;
  const int k0w = kt * BNK + 16 * w;
  const int j = k0w + n;

  bf16x8 kf[NKS], vf[NKS];   // B operands: K[j][32 ks + 8 g + e], V likewise
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const size_t off = (head + min(j, T - 1)) * D + 32 * ks + 8 * g;
    kf[ks] = *reinterpret_cast<const bf16x8*>(p.k + off);
    vf[ks] = *reinterpret_cast<const bf16x8*>(p.v + off);
  }
  f32x4 dv[NDB], dk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // per-lane byte offsets within a 32-row block of a tile (constant multiples of 32 rows
  // keep the swizzle): A-row reads per (half, k-step), transposed B reads per (d-block, half)
  uint32_t roff[2][NKS], toff[NDB][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int row = 8 * (n >> 2) + 4 * hf + (n & 3), chunk = 4 * ks + g;
      roff[hf][ks] = 16u * (uint32_t)(row * CPR + (chunk ^ swz16<CPR>(row)));
    }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 8 * g + ((lane >> 2) & 3) + 4 * hf, col = 16 * db + 4 * (lane & 3);
      toff[db][hf] = 2u * (uint32_t)(row * D + (((col >> 3) ^ swz16<CPR>(row)) << 3) + (col & 7));
    }

  const int i_start = kt * BNK;
  const int n_steps = (T - i_start + BMQ - 1) / BMQ;
  float lreg = 0.f, dreg = 0.f;
  auto load = [&](int st, Dkdv16Stage<D>& sm) {
    const int i0 = i_start + st * BMQ;
    tile_load16<CPR, BMQ>(sm.qs, [&](int row, int c) { return Q + (size_t)min(i0 + row, T - 1) * D + c * 8; });
    tile_load16<CPR, BMQ>(sm.gs, [&](int row, int c) { return G + (size_t)min(i0 + row, T - 1) * D + c * 8; });
    if (t < BMQ) {
      const int i = i0 + t;
      lreg = (i < T) ? p.lse[head + i] * kLog2e : __builtin_huge_valf();
      dreg = (i < T) ? p.delta[head + i] : 0.f;
    }
  };
  auto store_rows = [&](Dkdv16Stage<D>& sm) {
    if (t < BMQ) {
      sm.ls[t] = lreg;
      sm.dl[t] = dreg;
    }
  };
  auto lds_a = [](const bf16* tile, int qb, uint32_t off) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + qb * 32 * (CPR * 16) + off);
  };
  auto lds_b = [](const bf16* tile, int qb, uint32_t off_lo, uint32_t off_hi) {
    const char* base = reinterpret_cast<const char*>(tile) + qb * 32 * (CPR * 16);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_lo));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_hi));
    u32x4 r;
    r[0] = __builtin_bit_cast(u32x2, lo)[0];
    r[1] = __builtin_bit_cast(u32x2, lo)[1];
    r[2] = __builtin_bit_cast(u32x2, hi)[0];
    r[3] = __builtin_bit_cast(u32x2, hi)[1];
    return __builtin_bit_cast(bf16x8, r);
  };

  // one 32-query block: S, dP (two halves each), P and dS in registers, dV and dK.
  // `diag` marks the block on the diagonal: a query before this lane's key (query offset
  // 8 g + 4 h + r in the block, key offset 16 (w & 1) + n) gets zero weight.
  const int kdiag = 16 * (w & 1) + n;
  auto block = [&](const Dkdv16Stage<D>& sm, int qb, bool diag) {
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    pipelined<4 * NKS>(
        [&](int x) { return lds_a((x & 1) ? sm.gs : sm.qs, qb, roff[(x >> 1) & 1][x >> 2]); },
        [&](int x, const bf16x8& a) {
          const int hf = (x >> 1) & 1, ks = x >> 2;
          if (x & 1) dp[hf] = mfma16(a, vf[ks], dp[hf]);
          else sc[hf] = mfma16(a, kf[ks], sc[hf]);
        });
    float pr[8], dsr[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = qb * 32 + 8 * g + 4 * hf + r;
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hf][r], p.c, -sm.ls[qi]));
        if (diag && 8 * g + 4 * hf + r < kdiag) pv = 0.f;
        pr[4 * hf + r] = pv;
        dsr[4 * hf + r] = pv * (dp[hf][r] - sm.dl[qi]);
      }
    const bf16x8 pa = pack8(pr), da = pack8(dsr);
    // dV += P^T dO, dK += dS^T Q over the block's 32 queries (one 16x16x32 product each)
    pipelined<2 * NDB>([&](int x) { return lds_b((x & 1) ? sm.qs : sm.gs, qb, toff[x >> 1][0], toff[x >> 1][1]); },
                       [&](int x, const bf16x8& bop) {
                         if (x & 1) dk[x >> 1] = mfma16(da, bop, dk[x >> 1]);
                         else dv[x >> 1] = mfma16(pa, bop, dv[x >> 1]);
                       });
  };

  auto step = [&](int st, const Dkdv16Stage<D>& sm, Dkdv16Stage<D>& nxt) {
    if (st + 1 < n_steps) load(st + 1, nxt);
    if (st * BMQ < BNK) {
      // steps on the diagonal: 32-query block gq of the key tile meets this wave's keys
      // (16 w .. 16 w + 15 within the tile) for gq >= w / 2, and gq == w / 2 needs the mask
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) {
        const int gq = st * (BMQ / 32) + qb;
        if (gq < (w >> 1)) continue;
        block(sm, qb, gq == (w >> 1));
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < BMQ / 32; ++qb) block(sm, qb, false);
    }
    if (st + 1 < n_steps) store_rows(nxt);
    wait_vm0();
    __syncthreads();
  };

  load(0, stg[0]);
  store_rows(stg[0]);
  wait_vm0();
  __syncthreads();
  for (int st = 0; st < n_steps; st += 2) {  // unrolled by two: the LDS stage is a constant
    step(st, stg[0], stg[1]);
    if (st + 1 < n_steps) step(st + 1, stg[1], stg[0]);
  }

#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0w + 4 * g + r;
      if (key < T) {
        const size_t off = (head + key) * D + 16 * db + n;
        p.dv[off] = dv[db][r];
        p.dk[off] = dk[db][r] * p.scale;
      }
    }
}

// Both item kinds in one launch, heaviest key tile first: per key tile, the ordinary
// (b, h) items, then the frozen (h, column chunk) items.
template <int D>
__global__ __launch_bounds__(NTH16, 2) void dkdv_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[dkdv16_smem_bytes<D>()];
  const int kt = blockIdx.x / p.per_tile;
  int rem = blockIdx.x % p.per_tile;
  const int nd = p.B * p.n_dyn;
  if (rem < nd) {
    dkdv_dyn16<D>(p, rem / p.n_dyn, p.dyn[rem % p.n_dyn], kt, smem);
  } else {
    rem -= nd;
    dv_frz16<D>(p, p.frz[rem / p.n_chunks], rem % p.n_chunks, kt, smem);
  }
}

// ---------------------------------------------------------------- dQ

template <int D>
struct DqSmem {
  bf16 k[BND * D];    // K rows, swizzled; also read transposed
  bf16 v[BND * D];    // V rows, swizzled
};

template <int D>
__global__ __launch_bounds__(NTH, 2) void dq_kernel(const BwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * sizeof(DqSmem<D>)];
  DqSmem<D>* stg = reinterpret_cast<DqSmem<D>*>(smem_raw);
  const int item = blockIdx.x;
  const int n_qt = p.n_tiles;
  const int qt = n_qt - 1 - item / (p.B * p.n_dyn);
  const int bh = item % (p.B * p.n_dyn);
  const int b = bh / p.n_dyn, h = p.dyn[bh % p.n_dyn];
  const int lane = lane_id(), w = wave_id();
  const int m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const size_t head = ((size_t)b * p.H + h) * (size_t)T;
  const bf16* K = p.k + head * D;
  const bf16* V = p.v + head * D;
  const int i0w = qt * BMD + 32 * w, i = i0w + m;

  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = (head + min(i, T - 1)) * D + kk * 16 + hh * 8;
    qf[kk] = *reinterpret_cast<const bf16x8*>(p.q + off);
    gf[kk] = *reinterpret_cast<const bf16x8*>(p.dO + off);
  }
  const float lse2 = (i < T) ? p.lse[head + i] * kLog2e : __builtin_huge_valf();
  const float dlt = (i < T) ? p.delta[head + i] : 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const int n_kt = min(2 * qt + 2, (T + BND - 1) / BND);
  auto load = [&](int J, DqSmem<D>& sm) {
    const int j0 = J * BND;
    tile_load<CPR, BND>(sm.k, [&](int row, int c) { return K + (size_t)min(j0 + row, T - 1) * D + c * 8; });
    tile_load<CPR, BND>(sm.v, [&](int row, int c) { return V + (size_t)min(j0 + row, T - 1) * D + c * 8; });
  };

  uint32_t koff[D / 16], toff[NDB][2];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = row_off<CPR>(perm_rows(m), 2 * kk + hh);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    toff[db][0] = tr_off<CPR>(db * 32, 0, lane);
    toff[db][1] = tr_off<CPR>(db * 32, 1, lane);
  }

  auto tile = [&](int J, const DqSmem<D>& sm, DqSmem<D>& nxt) {
    if (J + 1 < n_kt) load(J + 1, nxt);
    const int j0 = J * BND;
    if (j0 <= i0w) {
      // per 32-key block: S^T = K Q^T and dP^T = V dO^T (two independent chains), then dS^T
      const bool diag = (j0 + BND - 1 > i0w);
      const int lim = i - j0 - 8 * hh;
      bf16x8 dsb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sd[2] = {f32x16{}, f32x16{}};   // 0: S^T, 1: dP^T
        pipelined<D / 8>(
            [&](int x) { return lds_row<CPR>((x & 1) ? sm.v : sm.k, kb * 32, koff[x >> 1]); },
            [&](int x, const bf16x8& a) { sd[x & 1] = mfma32(a, (x & 1) ? gf[x >> 1] : qf[x >> 1], sd[x & 1]); });
        float dsr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sd[0][r], p.c, -lse2));
          if (diag && kb * 32 + ((r >> 3) << 4) + (r & 7) > lim) pv = 0.f;
          dsr[r] = pv * (sd[1][r] - dlt);
        }
        dsb[2 * kb] = pack8(dsr);
        dsb[2 * kb + 1] = pack8(dsr + 8);
      }
      // dQ^T += K^T dS^T, K^T read transposed from the key tile
      pipelined<4 * NDB>([&](int x) { return lds_tr<CPR>(sm.k, (x / NDB) * 16, toff[x % NDB][0], toff[x % NDB][1]); },
                         [&](int x, const bf16x8& a) { acc[x % NDB] = mfma32(a, dsb[x / NDB], acc[x % NDB]); });
    }
    wait_vm0();
    __syncthreads();
  };

  load(0, stg[0]);
  wait_vm0();
  __syncthreads();
  for (int J = 0; J < n_kt; J += 2) {  // unrolled by two: the LDS stage is a constant
    tile(J, stg[0], stg[1]);
    if (J + 1 < n_kt) tile(J + 1, stg[1], stg[0]);
  }

  if (i < T) {
    float* out = p.dq + (head + i) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + acc_row(4 * g, hh);
        f32x4 v4;
        v4[0] = acc[db][4 * g] * p.scale;
        v4[1] = acc[db][4 * g + 1] * p.scale;
        v4[2] = acc[db][4 * g + 2] * p.scale;
        v4[3] = acc[db][4 * g + 3] * p.scale;
        *reinterpret_cast<f32x4*>(out + d) = v4;
      }
  }
}

BwdParams make_params(const AttnArgs& a, const void* q, const void* k, const void* v,
                      const void* dO, const float* lse, const float* delta, const float* alpha,
                      const float* rho, float* dq, float* dk, float* dv) {
  BwdParams p;
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.dO = static_cast<const bf16*>(dO);
  p.lse = lse;
  p.delta = delta;
  p.alpha = alpha;
  p.rho = rho;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.tab_stride = a.tab_stride;
  p.B = a.B;
  p.H = a.H;
  p.T = a.T;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.n_dyn = a.heads.n_dyn;
  p.n_frz = a.heads.n_frz;
  for (int x = 0; x < kMaxHeads; ++x) {
    p.dyn[x] = a.heads.dyn[x];
    p.frz[x] = a.heads.frz[x];
  }
  return p;
}

}  // namespace

hipError_t launch_delta(const AttnArgs& a, const void* o, const void* dO, float* delta,
                        hipStream_t s) {
  if (a.heads.n_dyn == 0) return hipSuccess;
  DeltaParams p;
  p.o = o;
  p.dO = dO;
  p.delta = delta;
  p.H = a.H;
  p.T = a.T;
  p.D = a.D;
  p.n_dyn = a.heads.n_dyn;
  p.n_rows = a.B * a.heads.n_dyn * a.T;
  p.bf16 = a.bf16;
  for (int x = 0; x < kMaxHeads; ++x) p.dyn[x] = a.heads.dyn[x];
  prof_begin("bwd_delta", s);
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((p.n_rows + 31) / 32), dim3(256), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const AttnArgs& a, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const float* alpha, const float* rho, float* dq, float* dk,
                           float* dv, float* delta, hipStream_t s) {
  hipError_t e = launch_delta(a, o, dO, delta, s);
  if (e != hipSuccess) return e;
  BwdParams p = make_params(a, q, k, v, dO, lse, delta, alpha, rho, dq, dk, dv);
  p.n_tiles = (a.T + BNK - 1) / BNK;
  p.n_chunks = (a.B * a.D + FCOLS - 1) / FCOLS;
  p.per_tile = a.B * p.n_dyn + p.n_frz * p.n_chunks;
  const int n_items = p.n_tiles * p.per_tile;
  if (n_items > 0) {
    prof_begin("dkdv", s);
    if (a.D == 64)
      hipLaunchKernelGGL(dkdv_kernel<64>, dim3(n_items), dim3(NTH16), 0, s, p);
    else
      hipLaunchKernelGGL(dkdv_kernel<128>, dim3(n_items), dim3(NTH16), 0, s, p);
    prof_end(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.n_dyn == 0) return hipSuccess;
  p.n_tiles = (a.T + BMD - 1) / BMD;
  const int n_dq = p.n_tiles * a.B * p.n_dyn;
  prof_begin("dq", s);
  if (a.D == 64)
    hipLaunchKernelGGL(dq_kernel<64>, dim3(n_dq), dim3(NTH), 0, s, p);
  else
    hipLaunchKernelGGL(dq_kernel<128>, dim3(n_dq), dim3(NTH), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
