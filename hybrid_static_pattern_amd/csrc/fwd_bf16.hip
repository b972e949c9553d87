// Hybrid causal attention forward, bf16 storage, fp32 accumulation, gfx950 MFMA.
//
// Method: "When Can Attention Heads Be Statically Defined?: 中文精读笔记".
//   ordinary head (part 一):  O = softmax_causal(scale Q K^T) V
//   frozen head (part 二.3, Eq. (3); part 二.4, Fig. 2):
//       O(i) = sum_{j<=i} exp(alpha(j) + rho(i-j)) V(j) / Z(i),
//       Z(i) = sum_{j<=i} exp(alpha(j) + rho(i-j))
// The page's fused kernel rebuilds a frozen tile from alpha, rho and Z and multiplies it
// by V, with ordinary heads on flash-style online-softmax tiles, in one launch per layer.
// Here both kinds of work items share one launch as well; the tiling is our own, built
// around 64-wide wavefronts and the 32x32x16 bf16 MFMA.
//
// A frozen row is a softmax over the logits alpha(j) + rho(i-j), so a frozen item runs the
// same online normaliser as an ordinary one, with the logits regenerated from alpha and
// rho (staged in LDS) instead of computed by Q K^T; log Z(i) comes out of it and is
// returned in lse for the backward. No separate pass over the T x T logits is needed.
//
// Work items (one 256-thread workgroup each, 4 waves x 32 queries = a 128-query tile):
//   dynamic (b, h, q-tile): S^T = K Q^T per 64-key tile (each lane keeps one query),
//       online softmax in log2 units with a lazy rescale (the running max is only raised
//       when a tile exceeds it by more than 2^8), O^T += V^T P^T;
//   frozen (h, q-tile, column chunk): the batch is folded into the columns, so one
//       item multiplies the regenerated pattern tile by up to 256 columns of
//       [V_0 | V_1 | ...] and the exp work is shared by every batch entry.
// Key tiles (and a frozen item's per-wave alpha / rho tables) go from HBM straight into one of
// NS LDS stages, NS - 1 tiles ahead of their use (no staging registers), one barrier per
// tile; V is stored row-major and read transposed (ds_read_b64_tr_b16). Two workgroups (three
// at D = 64 with 128 folded columns, four with 64) share a CU: their waves are not tied by a common
// barrier, so one runs its softmax arithmetic while another keeps the matrix cores busy. Items are issued heaviest q-tile first; key
// tiles above a wave's causal diagonal are skipped by that wave.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

constexpr int NW = 4;          // waves per workgroup
constexpr int BM = 32 * NW;    // queries per workgroup
constexpr int BN = 64;         // keys per tile
constexpr int NTH = 64 * NW;
constexpr int NS = 2;          // LDS stages
constexpr int FCOLS = 256;     // batch-folded columns per frozen item (at most)
constexpr int FTAB = 192;      // per-wave frozen table: alpha of the tile's keys, then rho

// -inf, read in place of table entries past the data (keys past T, negative distances)
__device__ float kNegSentinel[1] = {-__builtin_huge_valf()};
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
  int Hkv, G;  // key/value heads; query heads per key/value head
  float c;  // scale * log2(e)
  int n_dyn, n_frz, n_qt, n_chunks, per_qt;
  uint8_t dyn[kMaxHeads];
  uint8_t frz[kMaxHeads];
};

template <int D>
struct DynStage {
  bf16 k[BN * D];   // key tile, row-major, swizzled (swz<D/8>)
  bf16 v[BN * D];   // value tile, row-major, swizzled; read transposed
};

template <int FC>
struct FrzStage {
  bf16 v[BN * FC];        // folded value tile [key][column], swizzled; read transposed
  float tab[NW][FTAB];    // per wave: alpha of the tile's 64 keys, then rho over the wave's
                          // 95-distance window (-inf past the data)
};

// the frozen stage is sized by the launch's column count, so that narrow launches (D = 64 with
// at most 128 columns: 38 KiB instead of 70) fit three workgroups per CU
template <int D, int FC>
constexpr int smem_bytes() {
  return NS * (sizeof(DynStage<D>) > sizeof(FrzStage<FC>) ? (int)sizeof(DynStage<D>) : (int)sizeof(FrzStage<FC>));
}

// Online-softmax bookkeeping of one lane (one query row). `mx` is this lane's max over its
// logits of the tile (-inf where masked) and c converts logits to log2 units; the other
// half-wave holds the rest of the row. The running max m_used (log2 units) is raised
// lazily, and the accumulators are rescaled when it is. Returns the value to subtract
// before exp2: m_used, or 0 while no finite logit has been seen (then every exp2 of -inf
// is 0, never NaN).
template <int NACC>
__device__ __forceinline__ float online_rescale(float mx, float c, float& m_used, float& l,
                                                f32x16 (&acc)[NACC]) {
  mx = xhalf_max(mx) * c;
  const bool up = mx > m_used + kRescaleSlack;
  if (__any(up)) {
    const float m_new = up ? mx : m_used;
    const float a = (m_used == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_used - m_new);
#pragma unroll
    for (int x2 = 0; x2 < NACC; ++x2) acc[x2] *= a;
    l *= a;
    m_used = m_new;
  }
  return (m_used == kNegInf) ? 0.f : m_used;
}

// ---------------------------------------------------------------- dynamic item

template <int D>
__device__ void dyn_item(const FwdParams& p, int b, int h, int qt, unsigned char* smem_raw) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  DynStage<D>* st = reinterpret_cast<DynStage<D>*>(smem_raw);
  const int lane = lane_id(), w = wave_id();
  const int m = lane & 31, hh = lane >> 5;
  const int T = p.T;
  const size_t head = ((size_t)b * p.H + h) * (size_t)T;
  const size_t kv_head = ((size_t)b * p.Hkv + h / p.G) * (size_t)T;   // shared K/V of h's group
  const bf16* Q = p.q + head * D;
  const bf16* K = p.k + kv_head * D;
  const bf16* V = p.v + kv_head * D;
  const int i0w = qt * BM + w * 32;
  const int i = i0w + m;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(Q + (size_t)min(i, T - 1) * D + kk * 16 + hh * 8);

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_used = kNegInf, l = 0.f;

  // Key tiles are visited from the last one down, so that the two tiles that can hold a wave's
  // diagonal (BM = 2 BN) come first: they run in a peeled region with the causal mask, and
  // every later tile is a full one with no mask arithmetic.
  const int n_kt = min((qt + 1) * (BM / BN), (T + BN - 1) / BN);
  const RowTileLoader<CPR, BN, NW> rows;   // K and V tiles share their per-lane offsets
  auto load = [&](int s, int u) {
    const int J = max(n_kt - 1 - s, 0);   // steps past the end reload tile 0
    rows.load(st[u].k, K, J * BN, T);
    rows.load(st[u].v, V, J * BN, T);
  };
  // per-lane LDS offsets: K rows in pi order (one per k-step), V^T reads (per d-block)
  constexpr int NDB = D / 32;
  uint32_t koff[D / 16], voff[NDB][2];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = row_off<CPR>(perm_rows(m), 2 * kk + hh);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    voff[db][0] = tr_off<CPR>(db * 32, 0, lane);
    voff[db][1] = tr_off<CPR>(db * 32, 1, lane);
  }

  // one key tile; `diag` (the tile holding this wave's diagonal) masks keys after the query
  auto body = [&](const DynStage<D>& sm, int j0, bool diag) {
    // the compiler's MFMA / LDS-read interleaving strategy 0 for this region (alternating
    // runs on one box, 1B shape: forward 0.514 -> 0.507 ms; 124M and prefill shapes
    // unchanged; in the dQ kernel it was slower and is not used)
    __builtin_amdgcn_iglp_opt(0);
    {
      // S^T for keys j0 .. j0+63: two independent 32-key chains, interleaved
      f32x16 s[2] = {f32x16{}, f32x16{}};
      pipelined<D / 8>([&](int x) { return lds_row<CPR>(sm.k, (x & 1) * 32, koff[x >> 1]); },
                       [&](int x, const bf16x8& a) { s[x & 1] = mfma32(a, qf[x >> 1], s[x & 1]); });
      if (diag) {  // keys after the query get -inf
        const int lim = i - j0 - 8 * hh;  // key offset kb*32 + acc_pos(r, hh) > i - j0
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + ((r >> 3) << 4) + (r & 7) > lim) s[kb][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      const float msub = online_rescale<NDB>(mx, p.c, m_used, l, o);
      bf16x8 pb[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks >> 1][(ks & 1) * 8 + e], p.c, -msub));
          l += pv[e];
        }
        pb[ks] = pack8(pv);
      }
      // O^T += V^T P^T: the d-blocks are independent accumulators
      pipelined<4 * NDB>(
          [&](int x) { return lds_tr<CPR>(sm.v, (x / NDB) * 16, voff[x % NDB][0], voff[x % NDB][1]); },
          [&](int x, const bf16x8& a) { o[x % NDB] = mfma32(a, pb[x / NDB], o[x % NDB]); });
    }
  };
  auto tile = [&](int s, int u, bool peeled) {
    const int j0 = (n_kt - 1 - s) * BN;
    if (peeled) {
      if (j0 > i0w) return;  // the tile lies after this wave's queries
      body(st[u], j0, j0 + BN - 1 > i0w);
    } else {
      body(st[u], j0, false);
    }
  };
  constexpr int PERW = BN * CPR / (64 * NW);   // loads per wave and tile, for each of K, V
  static_assert(BM == 2 * BN && NS == 2, "the diagonal lies in the first two tiles visited");
  run_pipeline<NS, NS - 1, 2 * PERW, 2>(n_kt, load, tile, [&] {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) settle(qf[kk]);
  });

  const float lt = xhalf_sum(l);
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

// FC: folded columns per item (64, 128 or 256: B * D rounded up, at most 256)
template <int D, int FC>
__device__ void frz_item(const FwdParams& p, int h, int chunk, int qt, unsigned char* smem_raw) {
  constexpr int CPR = FC / 8;
  FrzStage<FC>* st = reinterpret_cast<FrzStage<FC>*>(smem_raw);
  const int lane = lane_id(), w = wave_id();
  const int m = lane & 31, hh = lane >> 5;
  const int T = p.T, H = p.H, B = p.B;
  const int col0 = chunk * FC;
  const int ncols = min(FC, B * D - col0);
  const int i0w = qt * BM + w * 32, i = i0w + m;
  const float* alpha = p.alpha + (size_t)h * p.tab_stride;
  const float* rho = p.rho + (size_t)h * p.tab_stride;

  // Columns past B*D (a partial last chunk) read clamped, valid data and are not stored.
  f32x16 o[FC / 32];
#pragma unroll
  for (int cb = 0; cb < FC / 32; ++cb) o[cb] = f32x16{};
  float m_used = kNegInf, l = 0.f;

  const int n_kt = min((qt + 1) * (BM / BN), (T + BN - 1) / BN);
  // this lane's chunks of each tile: folded column col0 + 8 chunk is column d of batch
  // element bb (columns past B * D, in a partial last chunk, read element B - 1 and are not
  // stored); 1 KiB block (w PERW + x) of the tile
  constexpr int PERW = BN * CPR / (64 * NW);
  // vrow[x]: this lane's chunk in row srow[x] of key tile 0 (V of h's key/value head)
  const bf16* vrow[PERW];
  int srow[PERW];
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int pch = (w * PERW + x) * 64 + lane, row = pch / CPR;
    const int col = col0 + ((pch % CPR) ^ swz<CPR>(row)) * 8;
    const int bb = min(col / D, B - 1), d = col % D;
    vrow[x] = p.v + (((size_t)bb * p.Hkv + h / p.G) * T + row) * D + d;
    srow[x] = row;
  }
  auto load = [&](int J, int u) {
    FrzStage<FC>& sm = st[u];
    const int j0 = J * BN;
    const bool full = j0 + BN <= T;
#pragma unroll
    for (int x = 0; x < PERW; ++x)
      // tiles with all 64 keys before T add j0 rows; the last one clamps rows to T - 1
      g2lds16(vrow[x] + (ptrdiff_t)(full ? j0 : min(j0 + srow[x], T - 1) - srow[x]) * D,
              lds_addr(sm.v) + (uint32_t)(w * PERW + x) * 1024u);
    // table entry e = 64 y + lane: alpha of key j0 + e (e < 64), then rho at distance
    // i0w - (j0 + 63) + (e - 64) (64 <= e < 159); -inf past the data
#pragma unroll
    for (int y = 0; y < FTAB / 64; ++y) {
      const int e = 64 * y + lane;
      const float* a = &kNegSentinel[0];
      if (e < BN) {
        if (full || j0 + e < T) a = alpha + j0 + e;
      } else if (e < 2 * BN + 31) {
        const int dd = i0w - (j0 + BN - 1) + (e - BN);
        if (dd >= 0) a = rho + min(dd, T - 1);
      }
      g2lds4(a, lds_addr(&sm.tab[w][64 * y]));
    }
  };

  uint32_t voff[FC / 32][2];
#pragma unroll
  for (int cb = 0; cb < FC / 32; ++cb) {
    voff[cb][0] = tr_off<CPR>(cb * 32, 0, lane);
    voff[cb][1] = tr_off<CPR>(cb * 32, 1, lane);
  }

  auto tile = [&](int J, int u, bool) {
    const FrzStage<FC>& sm = st[u];
    const int j0 = J * BN;
    if (j0 <= i0w) {
      // logits alpha(j) + rho(i - j); the window index of (i, j0 + kofs + e) is
      // m - (kofs + e) + 63, and entries for j > i hold -inf, so the causal mask comes for
      // free. The logits stay in registers between the max and the exps: all 32 of a tile
      // up to 128 columns, and next to the 128 accumulators of 256 columns the tile is taken
      // in two 32-key halves of 16 logits, each with its own max (an online softmax over any
      // split of the keys is exact).
      const float* tb = sm.tab[w];
      const int rb0 = BN + m + BN - 1 - hh * 8;
      auto logit = [&](int ks, int e) { return tb[ks * 16 + hh * 8 + e] + tb[rb0 - ks * 16 - e]; };
      constexpr int NHT = FC <= 128 ? 1 : 2;   // key halves of the tile
      constexpr int KSH = 4 / NHT;             // 16-key steps per half
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        float lg[KSH][8];
        float mx = kNegInf;
#pragma unroll
        for (int k2 = 0; k2 < KSH; ++k2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lg[k2][e] = logit(ht * KSH + k2, e);
            mx = fmaxf(mx, lg[k2][e]);
          }
        const float msub = online_rescale<FC / 32>(mx, kLog2e, m_used, l, o);
#pragma unroll
        for (int k2 = 0; k2 < KSH; ++k2) {
          const int ks = ht * KSH + k2;
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(lg[k2][e], kLog2e, -msub));
            l += pv[e];
          }
          const bf16x8 pb = pack8(pv);
          pipelined<FC / 32>([&](int cb) { return lds_tr<CPR>(sm.v, ks * 16, voff[cb][0], voff[cb][1]); },
                             [&](int cb, const bf16x8& a) { o[cb] = mfma32(a, pb, o[cb]); });
        }
      }
    }
  };
  run_pipeline<NS, NS - 1, PERW + FTAB / 64, 0>(n_kt, load, tile);

  const float lt = xhalf_sum(l);
  if (i < T) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int cb = 0; cb < FC / 32; ++cb) {
      if (cb * 32 >= ncols) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + cb * 32 + acc_row(4 * g, hh);
        const int bb = col / D, d = col % D;
        u32x2 pk;
        pk[0] = pack_bf16x2(o[cb][4 * g] * inv, o[cb][4 * g + 1] * inv);
        pk[1] = pack_bf16x2(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(p.o + (((size_t)bb * H + h) * T + i) * D + d) = pk;
      }
    }
    // log Z(i) is the same for every batch entry; the first column chunk writes it.
    if (chunk == 0 && hh == 0) {
      const float lz = (m_used + __log2f(lt)) * kLn2;
      for (int bb = 0; bb < B; ++bb) p.lse[((size_t)bb * H + h) * T + i] = lz;
    }
  }
}

// four workgroups per CU for D = 64 with at most 64 folded columns (124 registers), else two
// (three at D = 64 with 128 columns, by registers and LDS)
template <int D, int FC>
__global__ __launch_bounds__(NTH, (D == 64 && FC == 64) ? 4 : 2) void hybrid_fwd_kernel(const FwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[smem_bytes<D, FC>()];
  const int nd = p.B * p.n_dyn;
  int row, rem;
  if (!xcd_item(blockIdx.x, nd, p.n_frz * p.n_chunks, row, rem)) return;
  const int qt = p.n_qt - 1 - row;   // heaviest q-tile first
  if (rem < nd) {
    dyn_item<D>(p, rem / p.n_dyn, p.dyn[rem % p.n_dyn], qt, smem);
  } else {
    rem -= nd;
    frz_item<D, FC>(p, p.frz[rem / p.n_chunks], rem % p.n_chunks, qt, smem);
  }
}

}  // namespace

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
  p.Hkv = a.Hkv;
  p.G = a.G;
  p.c = a.scale * kLog2e;
  p.n_dyn = a.heads.n_dyn;
  p.n_frz = a.heads.n_frz;
  p.n_qt = (a.T + BM - 1) / BM;
  // folded columns per frozen item: B * D rounded up to 64, 128 or 256, except
  //  * D = 64: at most 128, so that the launch's LDS (the frozen stage is sized by the
  //    column count) fits three workgroups per CU, ordinary items included (alternating
  //    runs: 124M shape at r = 50% forward 0.258 -> 0.226 ms, B = 64 prefill shape at
  //    T = 2048 0.555 -> 0.526 ms);
  //  * D = 128 with at most a quarter of the heads frozen and B * D <= 512: 128 columns
  //    (more, narrower items between the ordinary ones, the logits kept in registers: 1B
  //    shape 0.510 -> 0.501 ms; with more frozen heads the regenerated pattern tiles
  //    dominate and 256 columns stay faster);
  //  * T <= 512: at most 128, where a few query tiles make a short grid whose critical path
  //    the longer 256-column items set.
  const bool narrow = a.D == 64 || (a.B * a.D <= 512 && 4 * a.heads.n_frz <= a.H) || a.T <= 512;
  int fc = a.B * a.D <= 64 ? 64 : (a.B * a.D <= 128 || narrow ? 128 : FCOLS);
  // a D = 64 launch without frozen heads takes the 64-column kernel, whose registers fit four
  // workgroups per CU (alternating runs, forward at r = 0: 124M shape 0.265 -> 0.257 ms,
  // B = 64 prefill shape at T = 2048 0.688 -> 0.637 ms); with frozen heads the 64-column
  // items cost more than the fourth workgroup gains (B = 64, T = 2048, r = 50%: 0.519 ->
  // 0.563 ms)
  if (a.D == 64 && a.heads.n_frz == 0) fc = 64;
  p.n_chunks = (a.B * a.D + fc - 1) / fc;
  p.per_qt = a.B * p.n_dyn + p.n_frz * p.n_chunks;
  for (int x = 0; x < kMaxHeads; ++x) {
    p.dyn[x] = a.heads.dyn[x];
    p.frz[x] = a.heads.frz[x];
  }
  const int n_items = p.n_qt * xcd_row_slots(a.B * p.n_dyn, p.n_frz * p.n_chunks);
  if (p.per_qt == 0) return hipSuccess;
  prof_begin("hybrid_fwd", s);
  const dim3 grid(n_items), block(NTH);
  if (a.D == 64) {   // narrow: at most 128 columns
    if (fc == 64) hipLaunchKernelGGL((hybrid_fwd_kernel<64, 64>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((hybrid_fwd_kernel<64, 128>), grid, block, 0, s, p);
  } else {
    if (fc == 128) hipLaunchKernelGGL((hybrid_fwd_kernel<128, 128>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((hybrid_fwd_kernel<128, FCOLS>), grid, block, 0, s, p);
  }
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
