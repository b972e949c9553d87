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
//   dq          ordinary (b, h, 128-query tile), keys from 0 to the diagonal, the query
//           as the lane index (as in the forward): dQ = scale * sum_J dS K_J. It runs
//           first because it also forms delta for its rows and writes it, with
//           lse * log2(e), for the dK/dV items;
//   dkdv        one launch of 4-wave workgroups on 16x16x32 MFMAs, two kinds of items:
//       ordinary (b, h, 128-key tile): each wave keeps 32 keys (K fragments and the fp32
//           dK, dV tiles) in registers and walks the 32-query steps from the diagonal
//           down; S and dP are computed with the key as the lane index so P and dS feed
//           the dV and dK products straight from registers;
//       frozen (h, 128-key tile, column chunk): the batch is folded into up to 256
//           columns of [dO_0 | dO_1 | ...]; P^T is regenerated per lane, rounded to fp16
//           (11 significant bits) and multiplied in one fp16 MFMA per tile by a copy of the
//           frozen heads' dO scaled by a power of two per (b, head) into fp16's range
//           (frz_half.hip, launched between dq and dkdv; dq's extra items take the block
//           maxima it needs), so the fp32 dV keeps P to 11 bits and dO exactly.
// bwd_delta forms delta on its own for the float32 path.
// Q/dO (dK/dV kernel) and K/V (dQ kernel) tiles go from HBM straight into multi-stage
// LDS, one barrier per step; the transposed operands (dO^T, Q^T, K^T) are read from the
// same row-major tiles with ds_read_b64_tr_b16. The split into a key-stationary and a
// query-stationary kernel recomputes S and dP once more instead of accumulating dQ with
// atomics (fp32 atomic adds run at about 1.3 TB/s on this GPU, and a fused kernel would issue
// gigabytes of them per layer); every output is written exactly once.
#include "frz_amax.h"
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

constexpr int BNK = 128;   // keys per dK/dV workgroup
constexpr int BMQ = 32;    // queries per dK/dV step
constexpr int NWD = 4;     // waves per dQ workgroup (two workgroups per CU)
constexpr int BMD = 32 * NWD;   // queries per dQ workgroup
constexpr int BND = 64;    // keys per dQ step
constexpr int NSD = 2;     // dQ LDS stages
constexpr int FCOLS = 256;   // batch-folded columns per frozen item (at most)

struct BwdParams {
  const bf16* o;        // forward output (the dQ kernel forms delta from it)
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dO;
  const float* lse;
  float* delta;         // delta_i of ordinary heads (written by the dQ kernel)
  float* ls2;           // lse * log2(e) of ordinary heads (written by the dQ kernel)
  const float* alpha;
  const float* rho;
  float* dq;
  float* dk;
  float* dv;
  FrzAmaxArgs famax;    // the frozen dO's block maxima, extra dQ items n_dq .. n_dq + n_famax - 1
  int n_dq, n_famax;
  const uint16_t* dh;   // frozen heads' dO in fp16, scaled per (b, frozen head): [B, n_frz, T, D]
  const int32_t* dexp;  // the scales' exponents [B * n_frz]: dV of batch b is 2^e times the product
  int tab_stride, B, H, T;
  int Hkv, G;   // key/value heads; query heads per key/value head
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
  const float* lse;
  float* ls2;   // lse * log2(e) (null: not written)
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
  if (row < p.n_rows && sub == 0) {
    p.delta[r] = acc;
    if (p.ls2) p.ls2[r] = p.lse[r] * kLog2e;
  }
}

// ---------------------------------------------------------------- dK / dV
//
// v_mfma_f32_16x16x32_bf16 throughout. Operand layout: A (16 x 32): lane l holds
// A[l % 16][8 (l / 16) + e]; B (32 x 16): lane l holds B[8 (l / 16) + e][l % 16]; C (16 x 16):
// lane l, register r holds C[4 (l / 16) + r][l % 16]. Below n = l % 16 and g = l / 16.
//
// One workgroup of 4 waves per 128-key tile; wave w owns keys 32 w .. 32 w + 31 (two 16-key
// groups kg) and keeps their K fragments and fp32 dK and dV tiles in registers, while the
// tile's V rows sit in LDS for the whole item. Every Q and dO byte a wave reads from LDS
// feeds two MFMAs. Steps are 32-query blocks whose Q / dO rows (and per-wave tables) go from
// HBM straight into one of NSK<D> LDS stages, NSK<D> - 1 steps ahead of their use. Small
// workgroups let two (D = 128) or three (D = 64) of them share a CU, their barriers
// independent (measured against one 8-wave workgroup per 256-key tile with four stages:
// 124M shape dK/dV 0.485 -> 0.396 ms, B = 64 prefill shape 0.889 -> 0.841 ms, 1B shape 1%).
//
// S = Q K^T is computed in two 16-query halves h whose A rows are the block's Q rows
// 8 (rho / 4) + 4 h + rho % 4 (rho = MFMA row): register r of half h in lane group g then
// holds query 8 g + 4 h + r, and the 8 values of lane group g are exactly the 8 consecutive
// queries 8 g .. 8 g + 7 that the P^T operand of the dV product needs (k index e = 4 h + r).

constexpr int NWK = 4;                   // waves per dK/dV workgroup
constexpr int NTK = 64 * NWK;
constexpr int KPW = BNK / NWK;           // keys per wave
constexpr int NKG = KPW / 16;            // 16-key groups per wave
// LDS stages: four for D = 64 (three workgroups per CU), two for D = 128 (two per CU)
template <int D> constexpr int NSK = D == 64 ? 4 : 2;
constexpr int DIAG_STEPS = BNK / BMQ;    // steps over the tile's own queries
static_assert(KPW == 32 && DIAG_STEPS % NSK<64> == 0 && DIAG_STEPS % NSK<128> == 0, "tile layout");

// Values read in place of rows past the data: +inf (a log-normaliser that zeroes its row's
// weights) and -inf (a distance table entry of a key after its query).
__device__ float kSentinel[2] = {__builtin_huge_valf(), -__builtin_huge_valf()};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Chunk swizzles. gfx950 serves ds_read_b128 in four groups of 16 lanes (the half-wave, and
// within it the parity of the lane's quad index (lane / 4) & 7) and ds_read_b64 /
// ds_read_b64_tr_b16 in half-waves, each group over 64 four-byte banks. hq = 0, 2, 3, 1 maps
// a 2-bit quad index so that the four quads of a b128 group get distinct values of
// g ^ hq(quad) and quads 2 m, 2 m + 1 differ in bit 1.
__device__ __forceinline__ int swz16_hq(int q) { return (((q ^ (q >> 1)) & 1) << 1) | (q >> 1); }
// Q and dO tiles (query rows), period 32 in the row. Reads:
//   A rows (b128): lane (n, g) reads row 8 (n / 4) + 4 h + n % 4, chunk 4 k + g;
//   B via ds_read_b64_tr_b16: lane l reads row 8 g + (l / 4) % 4 + 4 h, 8 bytes at
//   column 16 b + 4 (l % 4).
// Position bits 2-3 separate the four rows of a quad (row bits 0-1; for 128-byte rows, where
// row bit 0 already picks the bank half, row bit 1), and bits 0-1 take hq(row bits 3-4): the
// four quads of a b128 group then differ in chunk bits 0-1, and the two row blocks of a
// transposed half-wave in chunk bit 1. Row bit 2 is not used, so rows r and r + 4 share the
// swizzle, and k (bits 2-3 of the chunk) and b (bits 1-3) enter the byte offset as an XOR
// with 64 k and 32 b: a lane's offsets are one base XOR a constant.
template <int CPR>
__device__ __forceinline__ int swz16(int r) {
  return CPR >= 16 ? (((r & 3) << 2) | swz16_hq((r >> 3) & 3)) : ((((r >> 1) & 1) << 2) | swz16_hq((r >> 3) & 3));
}
// V tile (key rows), read as the B operand of dP = dO V^T: lane (n, g) reads row
// 16 m + n, chunk 4 k + g (b128). Same construction with hq taken from row bits 2-3.
template <int CPR>
__device__ __forceinline__ int swzv(int r) {
  return CPR >= 16 ? (((r & 3) << 2) | swz16_hq((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | swz16_hq((r >> 2) & 3));
}

// B operand (32 x 16) from a row-major query tile: two transposing reads, rows +0 and +4
template <int CPR>
__device__ __forceinline__ bf16x8 lds_b16(const bf16* tile, uint32_t off) {
  const char* base = reinterpret_cast<const char*>(tile);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off + 4 * CPR * 16));
  u32x4 r;
  r[0] = __builtin_bit_cast(u32x2, lo)[0];
  r[1] = __builtin_bit_cast(u32x2, lo)[1];
  r[2] = __builtin_bit_cast(u32x2, hi)[0];
  r[3] = __builtin_bit_cast(u32x2, hi)[1];
  return __builtin_bit_cast(bf16x8, r);
}
// 16-byte row read
__device__ __forceinline__ bf16x8 lds_16(const bf16* tile, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + off);
}
// per-lane byte offset of the transposed B read of column block 0, rows +0 (XOR 32 b for
// column block b)
template <int CPR>
__device__ __forceinline__ uint32_t tr16_base(int lane) {
  const int row = 8 * (lane >> 4) + ((lane >> 2) & 3), col = 4 * (lane & 3);
  return 2u * (uint32_t)(row * CPR * 8 + (((col >> 3) ^ swz16<CPR>(row)) << 3) + (col & 7));
}

template <int D>
struct DynStage {
  bf16 qs[BMQ * D];           // Q rows of the step, swizzled (swz16)
  bf16 gs[BMQ * D];           // dO rows of the step
  float tab[NWK][2 * BMQ];    // per wave: lse * log2(e) (+inf past T), then delta
};
template <int D>
struct DynSmem {
  DynStage<D> st[NSK<D>];
  bf16 vs[BNK * D];           // V rows of the key tile, swizzled (swzv)
};
template <int FC>
struct FrzStage {
  bf16 gs[BMQ * FC];          // folded dO [q][column], swizzled (swz16); read transposed
  float tab[NWK][128];        // per wave: log Z (+inf past T), then rho over the wave's
                              // 63-distance window (-inf for negative distances)
};

template <int D, int FC>
constexpr int dkdv_smem_bytes() {
  return sizeof(DynSmem<D>) > NSK<D> * sizeof(FrzStage<FC>) ? (int)sizeof(DynSmem<D>)
                                                            : (int)(NSK<D> * sizeof(FrzStage<FC>));
}

// Frozen item (h, 128-key tile, column chunk): dV_b[j] = sum_{i>=j} P(i,j) dO_b[i] for the
// batch folded into FC (64, 128 or 256) columns. Each wave keeps its 32 keys x FC columns of
// fp32 dV; P^T is regenerated per lane from alpha, rho and log Z (entries for j > i come out
// as 0 from the -inf distances of the window) and rounded to fp16, and the product takes the
// fp16 copy of dO scaled by 2^-e_bf (frz_half.hip): one fp16 MFMA per tile, P with 11
// significant bits, and dV_b scaled back by 2^e_bf when stored. f is h's frozen-head index.
template <int D, int FC>
__device__ void dv_frz(const BwdParams& p, int h, int f, int chunk, int kt, unsigned char* smem_raw) {
  constexpr int CPR = FC / 8;
  constexpr int NCB = FC / 16;
  // 16-byte chunks per lane per step: the 32 x FC tile splits evenly over the workgroup's
  // lanes (the same number of loads on every wave keeps the pipeline's counter waits uniform)
  static_assert(BMQ * CPR % NTK == 0, "frozen dO tile must split evenly over the lanes");
  constexpr int PERW = BMQ * CPR / NTK;
  FrzStage<FC>* stg = reinterpret_cast<FrzStage<FC>*>(smem_raw);
  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int T = p.T, H = p.H, B = p.B;
  const int col0 = chunk * FC;
  const int ncols = min(FC, B * D - col0);
  const int kbase = kt * BNK, k0w = kbase + KPW * w;
  const float* rho = p.rho + (size_t)h * p.tab_stride;
  float a2[NKG];
#pragma unroll
  for (int kg = 0; kg < NKG; ++kg) {
    const int j = k0w + 16 * kg + n;
    a2[kg] = (j < T) ? p.alpha[(size_t)h * p.tab_stride + j] * kLog2e : kNegInf;
  }

  f32x4 dv[NKG][NCB];
#pragma unroll
  for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) dv[kg][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t goff = tr16_base<CPR>(lane);

  // this lane's chunks of each step's tile: folded column col0 + 8 chunk is column d of batch
  // element bb (columns past B * D, in a partial last chunk, read element B - 1 and are not
  // stored); 1 KiB block (w PERW + x) of the tile
  // grow[x]: this lane's chunk in row kbase + srow[x] (step 0) of the folded dO
  const bf16* grow[PERW];
  int srow[PERW];
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int pch = (w * PERW + x) * 64 + lane, row = pch / CPR;
    const int col = col0 + ((pch % CPR) ^ swz16<CPR>(row)) * 8;
    const int bb = min(col / D, B - 1), d = col % D;
    grow[x] = reinterpret_cast<const bf16*>(p.dh) + (((size_t)bb * p.n_frz + f) * T + kbase + row) * D + d;
    srow[x] = row;
  }
  auto load = [&](int st, int u) {
    FrzStage<FC>& sm = stg[u];
    const int i0 = kbase + st * BMQ;
    const bool full = i0 + BMQ <= T;
#pragma unroll
    for (int x = 0; x < PERW; ++x)
      // steps with all 32 queries before T add their rows; the last ones clamp rows to T - 1
      g2lds16(grow[x] + (ptrdiff_t)(full ? st * BMQ : min(i0 + srow[x], T - 1) - kbase - srow[x]) * D,
              lds_addr(sm.gs) + (uint32_t)(w * PERW + x) * 1024u);
    // table entry e = 64 y + lane: log Z of query i0 + e (e < 32), then rho at distance
    // i0 - (k0w + 31) + e - 32 (32 <= e < 95)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int e = 64 * y + lane;
      const float* a;
      if (e < BMQ) {
        const int i = i0 + e;
        a = (i < T) ? p.lse + (size_t)h * T + i : &kSentinel[0];
      } else {
        const int dd = i0 - (k0w + KPW - 1) + (e - BMQ);
        a = (dd >= 0 && e < BMQ + BMQ + KPW - 1) ? rho + min(dd, T - 1) : &kSentinel[1];
      }
      g2lds4(a, lds_addr(&sm.tab[w][64 * y]));
    }
  };

  auto compute = [&](int st, int u, bool on_diag) {
    const FrzStage<FC>& sm = stg[u];
    if (on_diag && st < w) return;   // the block ends before this wave's keys
    const float* tb = sm.tab[w];
    // queries i0 + 8 g + e; window index of distance i - j is (8 g + e) - (16 kg + n) + 31
    const int qofs = 8 * g;
    f16x8 ap[NKG];
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
      const int rbase = BMQ + qofs - (16 * kg + n) + KPW - 1;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ap[kg][e] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(tb[rbase + e] - tb[qofs + e], kLog2e, a2[kg]));
    }
    pipelined<NCB>([&](int cb) { return lds_b16<CPR>(sm.gs, goff ^ (32u * cb)); },
                   [&](int cb, const bf16x8& bg) {
                     const f16x8 bh = __builtin_bit_cast(f16x8, bg);
#pragma unroll
                     for (int kg = 0; kg < NKG; ++kg)
                       dv[kg][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[kg], bh, dv[kg][cb], 0, 0, 0);
                   });
  };

  const int n_steps = (T - kbase + BMQ - 1) / BMQ;
  run_pipeline<NSK<D>, NSK<D> - 1, PERW + 2, DIAG_STEPS>(n_steps, load, compute, [&] {
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) settle(a2[kg]);
  });

#pragma unroll
  for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int col = col0 + 16 * cb + n;
      if (16 * cb >= ncols) continue;
      const int bb = col / D, d = col % D;
      const int e2 = p.dexp[bb * p.n_frz + f];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0w + 16 * kg + 4 * g + r;
        if (key < T) p.dv[(((size_t)bb * H + h) * T + key) * D + d] = ldexpf(dv[kg][cb][r], e2);
      }
    }
}

// Ordinary item (b, h, 128-key tile): dV and dK for the wave's 32 keys over all queries
// from the tile's first one to T, one 32-query block per step.
template <int D>
__device__ void dkdv_dyn(const BwdParams& p, int b, int h, int kt, unsigned char* smem_raw) {
  constexpr int CPR = D / 8;
  constexpr int NKS = D / 32;   // 32-wide k-steps over d
  constexpr int NDB = D / 16;   // 16-wide d blocks of dK, dV
  // waves 0..1 load the step's Q rows, waves 2..3 its dO rows
  constexpr int PERW = BMQ * CPR / (NTK / 2);
  constexpr int PERV = BNK * CPR / NTK;   // V tile chunks per lane
  static_assert(PERW >= 1 && PERV >= 1, "tile split");
  DynSmem<D>* smem = reinterpret_cast<DynSmem<D>*>(smem_raw);
  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int T = p.T;
  const size_t head = ((size_t)b * p.H + h) * (size_t)T;
  const size_t kv_head = ((size_t)b * p.Hkv + h / p.G) * (size_t)T;   // shared K/V of h's group
  const bf16* Q = p.q + head * D;
  const bf16* G = p.dO + head * D;
  const int kbase = kt * BNK, k0w = kbase + KPW * w;

  bf16x8 kf[NKG][NKS];   // B operands of S: K[j][32 ks + 8 g + e]
#pragma unroll
  for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kf[kg][ks] = *reinterpret_cast<const bf16x8*>(p.k + (kv_head + min(k0w + 16 * kg + n, T - 1)) * D + 32 * ks + 8 * g);
  // V rows of the key tile into LDS (rows past T re-read row T - 1; their keys are not stored)
#pragma unroll
  for (int x = 0; x < PERV; ++x) {
    const int pch = (w * PERV + x) * 64 + lane, row = pch / CPR;
    const int c = (pch % CPR) ^ swzv<CPR>(row);
    g2lds16(p.v + (kv_head + min(kbase + row, T - 1)) * D + c * 8, lds_addr(smem->vs) + (uint32_t)(w * PERV + x) * 1024u);
  }
  f32x4 dv[NKG][NDB], dk[NKG][NDB];
#pragma unroll
  for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dv[kg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dk[kg][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // per-lane byte offsets: A rows of half 0, k-step 0 (half h adds 4 rows, k-step k XORs
  // 64 k); the transposed B read of d-block 0 (d-block b XORs 32 b); the V read of key group
  // 0, k-step 0 (key group m adds 16 rows, k-step k XORs 64 k)
  const int arow = 8 * (n >> 2) + (n & 3);
  const uint32_t aoff = 16u * (uint32_t)(arow * CPR + (g ^ swz16<CPR>(arow)));
  const uint32_t boff = tr16_base<CPR>(lane);
  const int vrow = KPW * w + n;
  const uint32_t voff = 16u * (uint32_t)(vrow * CPR + (g ^ swzv<CPR>(vrow)));

  const bf16* tsrc = (w < NWK / 2) ? Q : G;
  const int wl = w & (NWK / 2 - 1);
  // per-lane offsets of a step's rows from its first row, and the lane's table entry (lanes
  // 0..31 lse * log2(e) of query lane, 32..63 delta) at step 0: for steps whose 32 queries all
  // lie before T the loads then cost no address arithmetic
  uint32_t roff[PERW];
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int pch = (wl * PERW + x) * 64 + lane, row = pch / CPR;
    roff[x] = 2u * (uint32_t)(row * D + ((pch % CPR) ^ swz16<CPR>(row)) * 8);
  }
  const float* tab0 = ((lane < 32) ? p.ls2 : p.delta) + head + kbase + (lane & 31);
  auto load = [&](int st, int u) {
    DynStage<D>& sm = smem->st[u];
    const int i0 = kbase + st * BMQ;
    bf16* tile = (w < NWK / 2) ? sm.qs : sm.gs;
    if (i0 + BMQ <= T) {
      const bf16* base = tsrc + (size_t)i0 * D;
#pragma unroll
      for (int x = 0; x < PERW; ++x) g2lds16_s(base, roff[x], lds_addr(tile) + (uint32_t)(wl * PERW + x) * 1024u);
      g2lds4(tab0 + st * BMQ, lds_addr(sm.tab[w]));
      return;
    }
    // rows past T (the last step, and the steps past the end) re-read row T - 1; the base row
    // ib <= every row read keeps the unsigned per-lane offsets non-negative
    const int ib = min(i0, T - 1);
#pragma unroll
    for (int x = 0; x < PERW; ++x) {
      const int pch = (wl * PERW + x) * 64 + lane, row = pch / CPR;
      const int c = (pch % CPR) ^ swz16<CPR>(row);
      const uint32_t o = 2u * (uint32_t)((min(i0 + row, T - 1) - ib) * D + c * 8);
      g2lds16_s(tsrc + (size_t)ib * D, o, lds_addr(tile) + (uint32_t)(wl * PERW + x) * 1024u);
    }
    // table: lanes 0..31 lse * log2(e) of query i0 + lane (+inf past T), lanes 32..63 delta
    const int i = i0 + (lane & 31);
    const float* a = (lane < 32) ? ((i < T) ? p.ls2 + head + i : &kSentinel[0]) : p.delta + head + min(i, T - 1);
    g2lds4(a, lds_addr(sm.tab[w]));
  };

  // One 32-query block: products() computes S and dP (two 16-query halves each) into sc, dp;
  // finish() turns them into P and dS in registers and accumulates dV and dK. On the block
  // that holds the wave's first key, a query before a lane's key (query offset 8 g + 4 h + r,
  // key offset 16 kg + n from the block start) gets S = -inf, so P = 0.
  f32x4 sc[NKG][2], dp[NKG][2];
  auto products = [&](const DynStage<D>& sm, bool diag) {
    // the compiler's interleaving strategy 0 for this region at D = 128 (alternating runs on
    // one box, 1B and grouped-query shapes: dK/dV 1% faster; at D = 64 it cost 12%)
    if constexpr (D == 128) __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        sc[kg][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kg][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // per k-step: NKG V reads (B of dP), then Q rows of halves 0, 1 and dO rows of halves 0, 1
    constexpr int PER = NKG + 4;
    bf16x8 vb[NKG];
    pipelined<PER * NKS>(
        [&](int x) {
          const int ks = x / PER, y = x % PER;
          if (y < NKG) return lds_16(smem->vs, (voff ^ (64u * ks)) + y * (16 * CPR * 16));
          const int hf = (y - NKG) & 1;
          return lds_16((y - NKG) >= 2 ? sm.gs : sm.qs, (aoff ^ (64u * ks)) + hf * (4 * CPR * 16));
        },
        [&](int x, const bf16x8& a) {
          const int ks = x / PER, y = x % PER;
          if (y < NKG) {
            vb[y] = a;
            return;
          }
          const int hf = (y - NKG) & 1;
#pragma unroll
          for (int kg = 0; kg < NKG; ++kg) {
            if ((y - NKG) >= 2) dp[kg][hf] = mfma16(a, vb[kg], dp[kg][hf]);
            else sc[kg][hf] = mfma16(a, kf[kg][ks], sc[kg][hf]);
          }
        });
    if (diag) {
#pragma unroll
      for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (8 * g + 4 * hf + r < 16 * kg + n) sc[kg][hf][r] = kNegInf;
    }
  };
  auto finish = [&](const DynStage<D>& sm) {
    const float* tb = sm.tab[w];
    bf16x8 pa[NKG], da[NKG];
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
      float pr[8], dsr[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qi = 8 * g + 4 * hf + r;
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kg][hf][r], p.c, -tb[qi]));
          pr[4 * hf + r] = pv;
          dsr[4 * hf + r] = pv * (dp[kg][hf][r] - tb[BMQ + qi]);
        }
      pa[kg] = pack8(pr);
      da[kg] = pack8(dsr);
    }
    // dV += P^T dO, dK += dS^T Q over the block's 32 queries
    pipelined<2 * NDB>([&](int x) { return lds_b16<CPR>((x & 1) ? sm.qs : sm.gs, boff ^ (32u * (x >> 1))); },
                       [&](int x, const bf16x8& bop) {
#pragma unroll
                         for (int kg = 0; kg < NKG; ++kg) {
                           if (x & 1) dk[kg][x >> 1] = mfma16(da[kg], bop, dk[kg][x >> 1]);
                           else dv[kg][x >> 1] = mfma16(pa[kg], bop, dv[kg][x >> 1]);
                         }
                       });
  };
  // block st meets this wave's keys iff 32 st + 31 >= 32 w; the block holding key 32 w is st = w
  auto compute = [&](int st, int u, bool on_diag) {
    if (on_diag && st < w) return;
    products(smem->st[u], on_diag && st == w);
    finish(smem->st[u]);
  };

  const int n_steps = (T - kbase + BMQ - 1) / BMQ;
  run_pipeline<NSK<D>, NSK<D> - 1, PERW + 1, DIAG_STEPS>(n_steps, load, compute, [&] {
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) settle(kf[kg][ks]);
  });

#pragma unroll
  for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0w + 16 * kg + 4 * g + r;
        if (key < T) {
          const size_t off = (head + key) * D + 16 * db + n;
          p.dv[off] = dv[kg][db][r];
          p.dk[off] = dk[kg][db][r] * p.scale;
        }
      }
}

// Both item kinds in one launch, heaviest key tile first: per key tile, the ordinary
// (b, h) items, then the frozen (h, column chunk) items.
template <int D, int FC>
__global__ __launch_bounds__(NTK, 2) void dkdv_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[dkdv_smem_bytes<D, FC>()];
  const int nd = p.B * p.n_dyn;
  int kt, rem;   // heaviest key tile (kt = 0) first
  if (!xcd_item(blockIdx.x, nd, p.n_frz * p.n_chunks, kt, rem)) return;
  if (rem < nd) {
    dkdv_dyn<D>(p, rem / p.n_dyn, p.dyn[rem % p.n_dyn], kt, smem);
  } else {
    rem -= nd;
    dv_frz<D, FC>(p, p.frz[rem / p.n_chunks], rem / p.n_chunks, rem % p.n_chunks, kt, smem);
  }
}

// ---------------------------------------------------------------- dQ

template <int D>
struct DqSmem {
  bf16 k[BND * D];    // K rows, swizzled; also read transposed
  bf16 v[BND * D];    // V rows, swizzled
};

template <int D>
__global__ __launch_bounds__(64 * NWD, 2) void dq_kernel(const BwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[NSD * sizeof(DqSmem<D>)];
  DqSmem<D>* stg = reinterpret_cast<DqSmem<D>*>(smem_raw);
  if ((int)blockIdx.x >= p.n_dq) {   // a block of the frozen dO's maxima (frz_amax.h)
    frz_amax_item(p.famax, p.frz, blockIdx.x - p.n_dq, reinterpret_cast<float*>(smem_raw));
    return;
  }
  int row, bh;
  if (!xcd_item(blockIdx.x, p.B * p.n_dyn, 0, row, bh)) return;
  const int qt = p.n_tiles - 1 - row;   // heaviest q-tile first
  const int b = bh / p.n_dyn, h = p.dyn[bh % p.n_dyn];
  const int lane = lane_id(), w = wave_id();
  const int m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const size_t head = ((size_t)b * p.H + h) * (size_t)T;
  const size_t kv_head = ((size_t)b * p.Hkv + h / p.G) * (size_t)T;   // shared K/V of h's group
  const bf16* K = p.k + kv_head * D;
  const bf16* V = p.v + kv_head * D;
  const int i0w = qt * BMD + 32 * w, i = i0w + m;

  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = (head + min(i, T - 1)) * D + kk * 16 + hh * 8;
    qf[kk] = *reinterpret_cast<const bf16x8*>(p.q + off);
    gf[kk] = *reinterpret_cast<const bf16x8*>(p.dO + off);
  }
  const float lse2 = (i < T) ? p.lse[head + i] * kLog2e : __builtin_huge_valf();
  // delta_i = sum_c dO_ic O_ic from this lane's half of the row (the dO fragments above) and
  // the other half-wave's; written with lse * log2(e) for the dK/dV kernel, which runs next
  float dlt = 0.f;
  {
    const bf16* orow = p.o + (head + min(i, T - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const bf16x8 of = *reinterpret_cast<const bf16x8*>(orow + kk * 16 + hh * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = __builtin_fmaf((float)of[e], (float)gf[kk][e], dlt);
    }
    dlt = xhalf_sum(dlt);
    if (i >= T) dlt = 0.f;
    if (i < T && hh == 0) {
      p.delta[head + i] = dlt;
      p.ls2[head + i] = lse2;
    }
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  // Key tiles are visited from the last one down, so that the two tiles that can hold a wave's
  // diagonal (BMD = 2 BND) come first: they run in a peeled region with the causal mask, and
  // every later tile is a full one with no mask arithmetic.
  const int n_kt = min((qt + 1) * (BMD / BND), (T + BND - 1) / BND);
  // K and V tiles share their per-lane offsets, kept in registers at D = 128 only: at D = 64
  // the two registers raise the kernel past 128 per lane, which costs a workgroup per CU
  // (alternating runs, 124M shape: dQ 0.239 -> 0.250 ms with them)
  const RowTileLoader<CPR, BND, NWD> rows;
  auto load = [&](int s, int u) {
    const int J = max(n_kt - 1 - s, 0);   // steps past the end reload tile 0
    if constexpr (D == 128) {
      rows.load(stg[u].k, K, J * BND, T);
      rows.load(stg[u].v, V, J * BND, T);
    } else {
      tile_load_rows<CPR, BND, NWD>(stg[u].k, K, J * BND, T);
      tile_load_rows<CPR, BND, NWD>(stg[u].v, V, J * BND, T);
    }
  };

  uint32_t koff[D / 16], toff[NDB][2];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = row_off<CPR>(perm_rows(m), 2 * kk + hh);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    toff[db][0] = tr_off<CPR>(db * 32, 0, lane);
    toff[db][1] = tr_off<CPR>(db * 32, 1, lane);
  }

  // one key tile; `diag` (the tile holding this wave's diagonal) zeroes keys after the query
  auto body = [&](const DqSmem<D>& sm, int j0, bool diag) {
    // per 32-key block: S^T = K Q^T and dP^T = V dO^T (two independent chains), then dS^T
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
  };
  auto tile = [&](int s, int u, bool peeled) {
    const int j0 = (n_kt - 1 - s) * BND;
    if (peeled) {
      if (j0 > i0w) return;  // the tile lies after this wave's queries
      body(stg[u], j0, j0 + BND - 1 > i0w);
    } else {
      body(stg[u], j0, false);
    }
  };
  constexpr int PERW = BND * CPR / (64 * NWD);   // loads per wave and tile, for each of K, V
  static_assert(BMD == 2 * BND && NSD == 2, "the diagonal lies in the first two tiles visited");
  run_pipeline<NSD, NSD - 1, 2 * PERW, 2>(n_kt, load, tile, [&] {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      settle(qf[kk]);
      settle(gf[kk]);
    }
  });

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
                      const void* dO, const float* lse, float* delta, const float* alpha,
                      const float* rho, float* dq, float* dk, float* dv) {
  BwdParams p;
  p.o = nullptr;
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
  p.dh = nullptr;
  p.dexp = nullptr;
  p.tab_stride = a.tab_stride;
  p.B = a.B;
  p.H = a.H;
  p.T = a.T;
  p.Hkv = a.Hkv;
  p.G = a.G;
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
                        const float* lse, float* ls2, hipStream_t s) {
  if (a.heads.n_dyn == 0) return hipSuccess;
  DeltaParams p;
  p.o = o;
  p.dO = dO;
  p.delta = delta;
  p.lse = lse;
  p.ls2 = ls2;
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
                           float* dv, float* delta, const FrzHalfWs& fh, hipStream_t s) {
  float* ls2 = delta + attn_ws_floats(a);
  BwdParams p = make_params(a, q, k, v, dO, lse, delta, alpha, rho, dq, dk, dv);
  p.dh = fh.dh;
  p.dexp = fh.dexp;
  p.o = static_cast<const bf16*>(o);
  p.ls2 = ls2;
  hipError_t e = hipSuccess;
  // dQ first: its items also write delta and lse * log2(e) of the ordinary rows, which the
  // dK/dV items read, and, as extra items after its own, the block maxima of the frozen heads'
  // dO; then the frozen dO in fp16 (frz_half.hip) for the frozen dK/dV items
  if (p.n_frz > 0) p.famax = frz_amax_args(a, dO, fh);
  p.n_famax = p.n_frz > 0 ? frz_half_blocks(a) * a.B * p.n_frz : 0;
  if (p.n_dyn > 0) {
    p.n_tiles = (a.T + BMD - 1) / BMD;
    p.n_dq = p.n_tiles * xcd_row_slots(a.B * p.n_dyn, 0);
    prof_begin("dq", s);
    if (a.D == 64)
      hipLaunchKernelGGL(dq_kernel<64>, dim3(p.n_dq + p.n_famax), dim3(64 * NWD), 0, s, p);
    else
      hipLaunchKernelGGL(dq_kernel<128>, dim3(p.n_dq + p.n_famax), dim3(64 * NWD), 0, s, p);
    prof_end(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_frz_half(a, dO, fh, p.n_dyn > 0, s)) != hipSuccess) return e;
  p.n_tiles = (a.T + BNK - 1) / BNK;
  // folded columns per frozen item: B * D rounded up to 64, 128 or 256, except at D = 64:
  // at most 128, so that the launch's LDS (the frozen stages are sized by the column count)
  // fits three workgroups per CU (alternating runs: 124M shape at r = 50% 0.380 -> 0.341 ms,
  // B = 64 prefill shape at T = 2048 0.828 -> 0.774 ms). Each item regenerates its pattern
  // tile, so wider items make fewer exps: with the single fp16 product per tile, 256 columns
  // beat 128 on the 1B shape at r = 25% too (dK/dV 0.819 -> 0.812 ms in alternating runs;
  // every head frozen: 0.45 vs 0.60 ms with the earlier two-product tile).
  const bool narrow = a.D == 64;
  const int fc = a.B * a.D <= 64 ? 64 : (a.B * a.D <= 128 || narrow ? 128 : FCOLS);
  p.n_chunks = (a.B * a.D + fc - 1) / fc;
  p.per_tile = a.B * p.n_dyn + p.n_frz * p.n_chunks;
  const int n_items = p.n_tiles * xcd_row_slots(a.B * p.n_dyn, p.n_frz * p.n_chunks);
  if (p.per_tile > 0) {
    prof_begin("dkdv", s);
    const dim3 grid(n_items), block(NTK);
    if (a.D == 64) {   // narrow: at most 128 columns
      if (fc == 64) hipLaunchKernelGGL((dkdv_kernel<64, 64>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dkdv_kernel<64, 128>), grid, block, 0, s, p);
    } else {
      if (fc == 128) hipLaunchKernelGGL((dkdv_kernel<128, 128>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dkdv_kernel<128, FCOLS>), grid, block, 0, s, p);
    }
    prof_end(s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace saf
