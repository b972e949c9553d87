// Calibration variance score, Eq. (1) of "When Can Attention Heads Be Statically Defined?:
// 中文精读笔记" (part 二.1): for each head, over N calibration sequences,
//     A_hat = (1/N) sum_n A^(n),   s_var = sum_n ||A^(n) - A_hat||_F^2 / ((N - 1) T^2),
// A^(n) = softmax_causal(scale Q_n K_n^T); heads are then ranked by ascending s_var.
//
// The T x T attention matrices are never stored. Three kernels:
//   var_lse      per (n, h, 128-query tile): the log2-domain row normaliser of every row
//                (max and sum over the causal keys, MFMA for Q K^T);
//   var_welford  per (h, 128-query tile, 64-key tile): loops over n, recomputes the tile
//                of A^(n) from Q_n, K_n and the row normaliser, and keeps Welford's running
//                mean and sum of squared deviations per entry in registers; writes the
//                A_hat tile and the tile's sum of squared deviations;
//   var_final    sums the per-tile partials in float64, divides by (N - 1) T^2 and ranks
//                the heads (stable: equal scores keep the lower head index first).
#include <type_traits>

#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

constexpr int NTH = 256;
constexpr int BM = 128;
constexpr int BN = 64;

struct VarParams {
  const bf16* q;
  const bf16* k;
  float* lse2;      // [N, H, T] log2 units
  float* partial;   // [H, n_it, n_jt]
  float* a_hat;
  double* s_var;
  int32_t* rank;
  int N, H, T;
  float c;          // scale * log2(e)
  float scale_n;    // scale / N (sharp mean)
  int n_it, n_jt;
};

template <int D>
struct KTile {
  bf16 k[BN * D];   // key rows, swizzled (swz<D/8>)
};

// One sequence's operands of a (128-query, 64-key) tile for the kernels that loop over the
// sequences: its key rows, its query rows and (Welford) the rows' normalisers, all loaded
// straight into LDS ahead of their use. Loading the query fragments into registers instead
// would make the wait for them (the counter of outstanding loads retires in order) also wait
// for the next sequence's tile loads issued before the use.
//
// The sequences go through two LDS stages, loaded one sequence ahead (50 KiB for D = 64:
// three workgroups per CU; a third stage measured slower, as it leaves room for two). Every
// wave issues the same number of loads per sequence (SEQ_LOADS<D> with the normalisers, one
// less without), so the wait for a stage is one counter value: waves 2 and 3 load the
// normalisers a second time into l2[BM..2 BM), which nothing reads.
template <int D>
struct SeqTile {
  bf16 k[BN * D];   // key rows, swizzled (swz<D/8>)
  bf16 q[BM * D];   // query rows, swizzled
  float l2[2 * BM]; // row normalisers, log2 units (rows past T repeat row T - 1)
};
constexpr int SEQ_STAGES = 2;
template <int D> constexpr int SEQ_LOADS = (BN + BM) * (D / 8) / NTH + 1;

// Tile index of workgroup b of G: XCD x (the one b % 8 runs on) takes a contiguous range of
// tiles, so the tiles of one head, which share query and key rows, share one L2 (measured:
// 0.28 -> 0.23 ms for the Welford pass at N = 64, H = 12, T = 1024; the tiles in grid order,
// spread over all eight L2s, fetch each query tile from memory up to eight times).
__device__ __forceinline__ int xcd_tile(int b, int G) {
  const int per = G / kNumXcd, rem = G % kNumXcd, x = b % kNumXcd;
  return x * per + min(x, rem) + b / kNumXcd;
}

// 4 bytes per lane from a wave-uniform base in SGPRs and a 32-bit per-lane byte offset:
// lane l's dword lands at lds_base + 4 l (as g2lds16_s, for the row normalisers).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void g2lds4_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase) : "m0");
}
#pragma clang diagnostic pop

// Per-lane byte offsets of a tile's loads within one sequence's [T, D] rows (and of its row
// normalisers within the [T] row): they depend on the tile and T only, so the loop over the
// sequences adds a wave-uniform base and spends no vector instructions on addresses.
template <int D>
struct SeqOffsets {
  static constexpr int CPR = D / 8;
  static constexpr int NK = BN * CPR / NTH, NQ = BM * CPR / NTH;   // loads per wave
  uint32_t k[NK], q[NQ], l2;
};

template <int CPR, int NR, int PERW>
__device__ __forceinline__ void tile_offsets(int r0, int T, uint32_t (&off)[PERW]) {
  static_assert(NR * CPR == PERW * NTH, "tile must split evenly over the waves");
  const int w = wave_id(), lane = lane_id();
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int pch = (w * PERW + x) * 64 + lane, row = pch / CPR;
    const int c = (pch % CPR) ^ swz<CPR>(row);
    off[x] = 2u * (uint32_t)(min(r0 + row, T - 1) * (CPR * 8) + c * 8);
  }
}

template <int D>
__device__ __forceinline__ SeqOffsets<D> seq_offsets(int i0, int j0, int T) {
  SeqOffsets<D> o;
  tile_offsets<D / 8, BN>(j0, T, o.k);
  tile_offsets<D / 8, BM>(i0, T, o.q);
  o.l2 = 4u * (uint32_t)min(i0 + 64 * (wave_id() & 1) + lane_id(), T - 1);
  return o;
}

// One sequence's tile loads with precomputed offsets: Q, K point at its [T, D] rows, l2 at its
// normalisers (all wave-uniform)
template <int D>
__device__ __forceinline__ void load_seq_off(const bf16* Q, const bf16* K, const float* l2, const SeqOffsets<D>& o,
                                             bool with_l2, SeqTile<D>& tile) {
  const int w = wave_id();
  const uint32_t kb = lds_addr(tile.k), qb = lds_addr(tile.q);
#pragma unroll
  for (int x = 0; x < SeqOffsets<D>::NK; ++x) g2lds16_s(K, o.k[x], kb + (uint32_t)(w * SeqOffsets<D>::NK + x) * 1024u);
#pragma unroll
  for (int x = 0; x < SeqOffsets<D>::NQ; ++x) g2lds16_s(Q, o.q[x], qb + (uint32_t)(w * SeqOffsets<D>::NQ + x) * 1024u);
  if (with_l2) g2lds4_s(l2, o.l2, lds_addr(&tile.l2[64 * w]));
}

// this lane's query fragments (row 32 w + m of the tile, k-halves hh) from LDS
template <int D>
__device__ __forceinline__ void lds_q(const SeqTile<D>& tile, int row, int hh, bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) qf[kk] = lds_row<D / 8>(tile.q, 0, row_off<D / 8>(row, 2 * kk + hh));
}

// S^T tile (64 keys x this lane's query) for the 64-key tile held in LDS; koff: per-lane
// offsets of the pi-ordered key rows, one per k-step.
template <int D>
__device__ __forceinline__ void scores(const bf16* ks, const bf16x8 (&qf)[D / 16], const uint32_t (&koff)[D / 16],
                                       f32x16 (&s)[2]) {
  s[0] = f32x16{};
  s[1] = f32x16{};
  pipelined<D / 8>([&](int x) { return lds_row<D / 8>(ks, (x & 1) * 32, koff[x >> 1]); },
                   [&](int x, const bf16x8& a) { s[x & 1] = mfma32(a, qf[x >> 1], s[x & 1]); });
}

template <int D>
__device__ __forceinline__ void key_offsets(int m, int hh, uint32_t (&koff)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = row_off<D / 8>(perm_rows(m), 2 * kk + hh);
}

template <int D>
__device__ __forceinline__ void load_q(const bf16* Q, int i, int T, int hh, bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Q + (size_t)min(i, T - 1) * D + kk * 16 + hh * 8);
}

// Row normalisers: key tiles go through LSE_STAGES LDS stages, three tiles ahead of their
// use, so a short item (a few tiles; the items are many) does not wait for each tile's load
// in turn. The running max is raised lazily (only when a tile's max exceeds it by more than
// 2^8 in log2 units), and the sum rescaled then, per lane and without a branch.
constexpr int LSE_STAGES = 4;
constexpr float kLseSlack = 8.0f;

template <int D>
__global__ __launch_bounds__(NTH, 2) void var_lse_kernel(const VarParams p) {
  __shared__ __attribute__((aligned(16))) KTile<D> stg[LSE_STAGES];
  const int n_qt = p.n_it;
  // heaviest query tiles first over the whole grid (an XCD-contiguous order, which shares
  // key rows through one L2 but ends on a tail of heavy tiles, measured 0.13 -> 0.17 ms)
  const int qt = n_qt - 1 - blockIdx.x / (p.N * p.H);
  const int nh = blockIdx.x % (p.N * p.H);
  const int lane = lane_id(), w = wave_id(), m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const size_t head = (size_t)nh * T;
  const int i0w = qt * BM + 32 * w, i = i0w + m;
  bf16x8 qf[D / 16];
  load_q<D>(p.q + head * D, i, T, hh, qf);
  uint32_t koff[D / 16];
  key_offsets<D>(m, hh, koff);
  const bf16* K = p.k + head * D;
  float m_run = kNegInf, l = 0.f;
  const int n_kt = min(2 * qt + 2, (T + BN - 1) / BN);
  const RowTileLoader<D / 8, BN, NTH / 64> rows;
  auto load = [&](int J, int u) {   // steps past the end reload the last tile (never used)
    rows.load(stg[u].k, K, min(J, n_kt - 1) * BN, T);
  };
  constexpr int PERW = BN * (D / 8) / NTH;
  auto body = [&](int j0, int u, auto diag_t) {
    f32x16 s[2];
    scores<D>(stg[u].k, qf, koff, s);
    if constexpr (decltype(diag_t)::value) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + kb * 32 + acc_pos(r, hh) > i) s[kb][r] = kNegInf;
    }
    // a chain of max3 (a balanced tree of fmaxf canonicalises every MFMA result first)
    float mx = kNegInf;
#pragma unroll
    for (int x = 0; x < 32; ++x) mx = fmaxf(mx, s[x >> 4][x & 15]);
    mx = xhalf_max(mx) * p.c;
    const bool up = mx > m_run + kLseSlack;
    const float m_new = up ? mx : m_run;
    // m_run = -inf on the first tile: the factor is exp2(-inf) = 0 and l starts from 0
    l *= up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    m_run = m_new;
    float e[32];
#pragma unroll
    for (int x = 0; x < 32; ++x) e[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x >> 4][x & 15], p.c, -m_run));
    l += tree_sum<32>(e);
  };
  // the causal mask only on the tiles that hold a wave's diagonal (a branch, not selects)
  auto tile = [&](int J, int u, bool) {
    const int j0 = J * BN;
    if (j0 > i0w) return;
    if (j0 + BN - 1 > i0w) body(j0, u, std::true_type{});
    else body(j0, u, std::false_type{});
  };
  run_pipeline<LSE_STAGES, LSE_STAGES - 1, PERW, 0>(n_kt, load, tile, [&] {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) settle(qf[kk]);
  });
  const float lt = xhalf_sum(l);
  if (i < T && hh == 0) p.lse2[head + i] = m_run + __log2f(lt);
}

// KL = false: Welford's mean and M2, the tile's partial is sum M2 (Eq. (1)).
// KL = true: the mean and, per lane, sum_n a log2 a (log2 a is the exponent itself); the
// tile's partial is ln 2 [sum_n sum a log2 a / N - sum A_hat log2 A_hat], its share of
// N T s^KL / N: since sum_n A^(n) = N A_hat entrywise,
// sum_n KL(A^(n)_i || A_hat_i) = sum_n sum_j A^(n) log A^(n) - N sum_j A_hat log A_hat.
template <int D, bool KL>
__global__ __launch_bounds__(NTH, 2) void var_welford_kernel(const VarParams p) {
  constexpr int NS = SEQ_STAGES;
  __shared__ __attribute__((aligned(16))) SeqTile<D> stg[NS];
  __shared__ float red[NTH / 64];
  // Work order: the tiles every wave works on (jt <= 2 it: it^2 per head) first, in contiguous
  // ranges per XCD so that one head's query and key rows share an L2; then the tiles right
  // of the diagonal block (jt = 2 it + 1, where two of the four waves have no causal entry:
  // half the work), so that the last round of workgroups is a light one; then one workgroup per
  // row band for the zeros above the diagonal.
  const int n_full = p.H * p.n_it * p.n_it;
  const int n_half = (p.n_jt >= 2 * p.n_it) ? p.n_it : p.n_it - 1;
  int h, it, jt;
  if ((int)blockIdx.x < n_full) {
    const int tile = xcd_tile(blockIdx.x, n_full), e = tile % (p.n_it * p.n_it);
    h = tile / (p.n_it * p.n_it);
    it = (int)sqrtf((float)e);
    while (it * it > e) --it;
    while ((it + 1) * (it + 1) <= e) ++it;
    jt = e - it * it;
  } else if ((int)blockIdx.x < n_full + p.H * n_half) {
    const int x = blockIdx.x - n_full;
    h = x / n_half;
    it = x % n_half;
    jt = 2 * it + 1;
  } else {
    const int x = blockIdx.x - n_full - p.H * n_half;
    h = x / p.n_it;
    it = x % p.n_it;
    jt = -1;
  }
  const int t = threadIdx.x, lane = lane_id(), w = wave_id(), m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const int i0 = it * BM, i0w = i0 + 32 * w, i = i0w + m, j0 = jt * BN;
  float* A = p.a_hat + (size_t)h * T * T;

  if (jt < 0) {   // row band it above the diagonal block: A_hat is 0 there, partials are 0
    const int c0 = (2 * it + 2) * BN;   // first column to the right of the diagonal block
    const int w4 = (T - c0 + 3) / 4;    // 4-column groups per row (the last may be partial)
    for (int x = t; x < BM * max(w4, 0); x += NTH) {
      const int r = x / w4, ii = i0 + r, jj = c0 + 4 * (x % w4);
      if (ii >= T) continue;
      if ((T & 3) == 0) {
        *reinterpret_cast<f32x4*>(A + (size_t)ii * T + jj) = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        for (int e = 0; e < 4; ++e)
          if (jj + e < T) A[(size_t)ii * T + jj + e] = 0.f;
      }
    }
    for (int x = 2 * it + 2 + t; x < p.n_jt; x += NTH) p.partial[((size_t)h * p.n_it + it) * p.n_jt + x] = 0.f;
    return;
  }
  float* part = p.partial + ((size_t)h * p.n_it + it) * p.n_jt + jt;

  float mean[32], m2[KL ? 1 : 32];
  float alog = 0.f;   // KL: sum over n and this lane's entries of a log2 a
#pragma unroll
  for (int x = 0; x < 32; ++x) {
    mean[x] = 0.f;
    if constexpr (!KL) m2[x] = 0.f;
  }
  const bool active = j0 <= i0w;     // wave has causal entries in this tile
  const bool diag = j0 + BN - 1 > i0w;
  const size_t nh_stride = (size_t)p.H * T;
  uint32_t koff[D / 16];
  key_offsets<D>(m, hh, koff);
  const SeqOffsets<D> goff = seq_offsets<D>(i0, j0, T);
  auto load = [&](int n, int u) {  // sequences past N re-read the last one (never used)
    const size_t head = (size_t)min(n, p.N - 1) * nh_stride + (size_t)h * T;
    load_seq_off<D>(p.q + head * D, p.k + head * D, p.lse2 + head, goff, true, stg[u]);
  };
  run_pipeline<NS, NS - 1, SEQ_LOADS<D>, 0>(p.N, load, [&](int n, int u, bool) {
    if (active) {
      const SeqTile<D>& cur = stg[u];
      bf16x8 qf[D / 16];
      lds_q<D>(cur, 32 * w + m, hh, qf);
      const float l2 = (i < T) ? cur.l2[32 * w + m] : __builtin_huge_valf();
      f32x16 s[2];
      scores<D>(cur.k, qf, koff, s);
      // 1 / (n + 1) by the hardware reciprocal (within 1 ulp; exact for n = 0, so N equal
      // sequences still leave M2 = 0 exactly)
      const float rn = __builtin_amdgcn_rcpf((float)(n + 1));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = __builtin_fmaf(s[kb][r], p.c, -l2);
          float a = __builtin_amdgcn_exp2f(z);
          const int x = kb * 16 + r;
          if constexpr (KL) {
            if (diag && j0 + kb * 32 + acc_pos(r, hh) > i) a = 0.f;
            if (a > 0.f) alog = __builtin_fmaf(a, z, alog);
          }
          // Welford: entries after the query (diagonal tiles) accumulate whatever their
          // logits give and are set to 0 once after the loop, which is the same as feeding
          // them zeros, since every entry's mean and M2 are its own
          const float dlt = a - mean[x];
          mean[x] = __builtin_fmaf(dlt, rn, mean[x]);
          if constexpr (!KL) m2[x] = __builtin_fmaf(dlt, a - mean[x], m2[x]);
        }
    }
  });
  if (diag) {   // entries after the query: A_hat = 0 and no deviation
#pragma unroll
    for (int x = 0; x < 32; ++x)
      if (j0 + (x >> 4) * 32 + acc_pos(x & 15, hh) > i) {
        mean[x] = 0.f;
        if constexpr (!KL) m2[x] = 0.f;
      }
  }

  float sum = 0.f;
  if (i < T) {
    float* row = A + (size_t)i * T;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sk = 0; sk < 2; ++sk) {
        const int jj = j0 + kb * 32 + sk * 16 + hh * 8;
        const float* mv = mean + kb * 16 + sk * 8;
        if ((T & 3) == 0 && jj + 7 < T) {
          *reinterpret_cast<f32x4*>(row + jj) = f32x4{mv[0], mv[1], mv[2], mv[3]};
          *reinterpret_cast<f32x4*>(row + jj + 4) = f32x4{mv[4], mv[5], mv[6], mv[7]};
        } else {
          for (int e = 0; e < 8; ++e)
            if (jj + e < T) row[jj + e] = mv[e];
        }
      }
    if constexpr (KL) {
      float hl = 0.f;
#pragma unroll
      for (int x = 0; x < 32; ++x)
        if (mean[x] > 0.f) hl = __builtin_fmaf(mean[x], __log2f(mean[x]), hl);
      sum = kLn2 * (alog / (float)p.N - hl);
    } else {
#pragma unroll
      for (int x = 0; x < 32; ++x) sum += m2[x];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  if (t == 0) *part = red[0] + red[1] + red[2] + red[3];
}

// Sums each head's tile partials in float64 and ranks the heads by the score:
// KL = false: s_var = sum M2 / ((N - 1) T^2); KL = true: s^KL = sum / T.
template <bool KL>
__global__ __launch_bounds__(256) void var_final_kernel(const VarParams p) {
  __shared__ double sv[kMaxHeads];
  const int h = threadIdx.x;
  const int per = p.n_it * p.n_jt;
  // each wave sums the partials of heads w, w + 4, ...: its lanes take every 64th partial,
  // then a butterfly over the wave (the loads of one head are independent, not a chain)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int hh = wv; hh < p.H; hh += 4) {
    const float* part = p.partial + (size_t)hh * per;
    double acc = 0.0;
    for (int x = lane; x < per; x += 64) acc += (double)part[x];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) {
      const double v = KL ? acc / (double)p.T : acc / ((double)(p.N - 1) * (double)p.T * (double)p.T);
      sv[hh] = v;
      p.s_var[hh] = v;
    }
  }
  __syncthreads();
  if (h < p.H) {
    const double v = sv[h];
    int pos = 0;
    for (int x = 0; x < p.H; ++x) pos += (sv[x] < v) || (sv[x] == v && x < h);
    p.rank[pos] = h;
  }
}

// Sharp mean (part 二.2): the logits are averaged over the N sequences first,
// P_sharp = softmax_causal((1/N) sum_n scale Q_n K_n^T). sharp_logits_kernel accumulates the
// S^T tile of every n in the same MFMA accumulators (K-dimension N D) and writes the mean
// logits of the tile's causal entries into `out`; sharp_rows_kernel then turns each row into
// its causal softmax in place and writes the zeros above the diagonal.
template <int D>
__global__ __launch_bounds__(NTH, 2) void sharp_logits_kernel(const VarParams p, float* out) {
  constexpr int NS = SEQ_STAGES;
  __shared__ __attribute__((aligned(16))) SeqTile<D> stg[NS];
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int jt = tile % p.n_jt;
  const int it = (tile / p.n_jt) % p.n_it;
  const int h = tile / (p.n_jt * p.n_it);
  const int lane = lane_id(), w = wave_id(), m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const int i0 = it * BM, i0w = i0 + 32 * w, i = i0w + m, j0 = jt * BN;
  if (j0 > i0 + BM - 1) return;   // above the diagonal: written by the row kernel
  const bool active = j0 <= i0w;
  const size_t nh_stride = (size_t)p.H * T;
  uint32_t koff[D / 16];
  key_offsets<D>(m, hh, koff);
  const SeqOffsets<D> goff = seq_offsets<D>(i0, j0, T);
  auto load = [&](int n, int u) {  // sequences past N re-read the last one (never used)
    const size_t head = (size_t)min(n, p.N - 1) * nh_stride + (size_t)h * T;
    load_seq_off<D>(p.q + head * D, p.k + head * D, nullptr, goff, false, stg[u]);
  };
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  run_pipeline<NS, NS - 1, SEQ_LOADS<D> - 1, 0>(p.N, load, [&](int n, int u, bool) {
    if (active) {
      bf16x8 qf[D / 16];
      lds_q<D>(stg[u], 32 * w + m, hh, qf);
      pipelined<D / 8>([&](int x) { return lds_row<D / 8>(stg[u].k, (x & 1) * 32, koff[x >> 1]); },
                       [&](int x, const bf16x8& a) { acc[x & 1] = mfma32(a, qf[x >> 1], acc[x & 1]); });
    }
  });
  if (!active || i >= T) return;
  const float f = p.scale_n;
  float* row = out + ((size_t)h * T + i) * T;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int sk = 0; sk < 2; ++sk) {
      const int jj = j0 + kb * 32 + sk * 16 + hh * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (jj + e <= i) row[jj + e] = acc[kb][sk * 8 + e] * f;
    }
}

// one wave per row i: max and sum over j <= i of the mean logits, then the row in place
__global__ __launch_bounds__(256) void sharp_rows_kernel(int H, int T, float* out) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), h = blockIdx.y;
  if (i >= T) return;
  float* row = out + ((size_t)h * T + i) * T;
  float mx = -__builtin_huge_valf();
  for (int j = lane; j <= i; j += 64) mx = fmaxf(mx, row[j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float sum = 0.f;
  for (int j = lane; j <= i; j += 64) sum += __builtin_amdgcn_exp2f((row[j] - mx) * kLog2e);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  const float inv = 1.f / sum;
  for (int j = lane; j < T; j += 64) row[j] = j <= i ? __builtin_amdgcn_exp2f((row[j] - mx) * kLog2e) * inv : 0.f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t var_workspace_bytes(const VarArgs& a) {
  const size_t n_it = (a.T + BM - 1) / BM, n_jt = (a.T + BN - 1) / BN;
  return align256((size_t)a.N * a.H * a.T * sizeof(float)) + align256((size_t)a.H * n_it * n_jt * sizeof(float));
}

hipError_t launch_sharp_mean(const VarArgs& a, const void* q, const void* k, float* out, hipStream_t s) {
  VarParams p{};
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.N = a.N;
  p.H = a.H;
  p.T = a.T;
  p.scale_n = a.scale / (float)a.N;
  p.n_it = (a.T + BM - 1) / BM;
  p.n_jt = (a.T + BN - 1) / BN;
  prof_begin("sharp_logits", s);
  if (a.D == 64)
    hipLaunchKernelGGL(sharp_logits_kernel<64>, dim3(p.n_jt * p.n_it * a.H), dim3(NTH), 0, s, p, out);
  else
    hipLaunchKernelGGL(sharp_logits_kernel<128>, dim3(p.n_jt * p.n_it * a.H), dim3(NTH), 0, s, p, out);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin("sharp_rows", s);
  hipLaunchKernelGGL(sharp_rows_kernel, dim3((a.T + 3) / 4, a.H), dim3(256), 0, s, a.H, a.T, out);
  prof_end(s);
  return hipGetLastError();
}

hipError_t launch_var_score(const VarArgs& a, const void* q, const void* k, float* a_hat,
                            double* s_var, int32_t* rank, void* ws, hipStream_t s, bool kl) {
  VarParams p;
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.lse2 = static_cast<float*>(ws);
  p.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)a.N * a.H * a.T * sizeof(float)));
  p.a_hat = a_hat;
  p.s_var = s_var;
  p.rank = rank;
  p.N = a.N;
  p.H = a.H;
  p.T = a.T;
  p.c = a.scale * kLog2e;
  p.n_it = (a.T + BM - 1) / BM;
  p.n_jt = (a.T + BN - 1) / BN;
  prof_begin("var_lse", s);
  if (a.D == 64)
    hipLaunchKernelGGL(var_lse_kernel<64>, dim3(p.n_it * a.N * a.H), dim3(NTH), 0, s, p);
  else
    hipLaunchKernelGGL(var_lse_kernel<128>, dim3(p.n_it * a.N * a.H), dim3(NTH), 0, s, p);
  prof_end(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // full tiles, half tiles right of each diagonal block, one zero-writer per row band
  const int n_half = (p.n_jt >= 2 * p.n_it) ? p.n_it : p.n_it - 1;
  const dim3 grid(a.H * (p.n_it * p.n_it + n_half + p.n_it)), block(NTH);
  prof_begin(kl ? "kl_welford" : "var_welford", s);
  if (a.D == 64) {
    if (kl) hipLaunchKernelGGL((var_welford_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((var_welford_kernel<64, false>), grid, block, 0, s, p);
  } else {
    if (kl) hipLaunchKernelGGL((var_welford_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((var_welford_kernel<128, false>), grid, block, 0, s, p);
  }
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin("var_final", s);
  if (kl) hipLaunchKernelGGL(var_final_kernel<true>, dim3(1), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(var_final_kernel<false>, dim3(1), dim3(256), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
