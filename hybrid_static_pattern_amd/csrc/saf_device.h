// Device-side building blocks shared by the libsaf kernels (gfx950 / CDNA4).
//
// MFMA tile convention (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16):  lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32):  lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32):  lane l, accumulator r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// Every attention product here is arranged so that the output column (l % 32) is the
// index a lane keeps for the whole tile (a query in the forward, a key in the backward),
// which turns row-wise softmax statistics into per-lane scalars.
//
// Row permutation pi: when a C tile is later fed back as the B (or A) operand of a second
// product, lane half h must hold 8 consecutive positions of the contracted index. The C
// rows a lane holds are {8(r/4) + 4h + r%4}; loading the first product's A rows in the
// order pi(m) = m with bits 2 and 3 swapped makes accumulator r of lane half h hold
// position 16(r/8) + 8h + r%8, i.e. k-step r/8, element r%8.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index, known to the compiler as wave-uniform (scalar register)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// bits 2 and 3 of m swapped (an involution on 0..31)
__device__ __forceinline__ int perm_rows(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Position (0..31) within a 32-block held by accumulator r of lane half h after the
// pi-ordered product, see the header comment.
__device__ __forceinline__ int acc_pos(int r, int h) { return ((r >> 3) << 4) + (h << 3) + (r & 7); }

// Row of a C tile held by accumulator r of lane half h (no permutation).
__device__ __forceinline__ int acc_row(int r, int h) { return ((r >> 2) << 3) + (h << 2) + (r & 3); }

// LDS swizzles (16-byte chunk index XOR a 3-bit row function). A row of a
// "row-major" tile holds the contracted index contiguously; reads of one 16-byte chunk
// by 8 consecutive lanes then fall on distinct chunks.
// Rows read in pi order (rows {0,1,2,3,8,9,10,11}+...): use bits 0,1,3 of the row.
__device__ __forceinline__ int swz_pi(int row) { return (row & 3) | ((row >> 1) & 4); }
// Rows read consecutively and written 8 apart (transposed staging): bits 0-2 ^ bits 3-5.
__device__ __forceinline__ int swz_tr(int row) { return (row ^ (row >> 3)) & 7; }

// ---------------------------------------------------------------- LDS tiles
//
// A tile is row-major in LDS, CPR 16-byte chunks per row, and chunk c of row r is stored
// at position c ^ swz<CPR>(r). Two read patterns use the same tiles:
//   * ds_read_b128 of rows in pi order (an MFMA A operand whose rows are the tile rows):
//     16 consecutive lanes read rows {0,1,2,3,8,9,10,11,4,5,6,7,12,13,14,15} (+16) at one
//     logical chunk;
//   * ds_read_b64_tr_b16 (an operand whose rows are the tile columns, see lds_tr_operand):
//     lanes 0-31 read rows 0..3 and lanes 32-63 rows 8..11 (+ base), 64 bytes each.
// With 64 four-byte banks (256 bytes per cycle) the swizzle puts the 16 rows of the first
// pattern on 16 distinct chunk positions, and the four rows of each half-wave of the second
// on four distinct 64-byte groups. 256-byte rows (CPR 16) all start at bank 0; 128-byte
// rows (CPR 8) alternate between the two bank halves.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  return CPR >= 16 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// element offset of (row, col) in a swizzled tile with CPR chunks per row
template <int CPR>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * (CPR * 8) + ((((col >> 3) ^ swz<CPR>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// Global -> LDS without registers: lane l's 16 bytes at gsrc land at LDS byte address
// lds_base + 16 l (lds_base wave-uniform). Issued through inline assembly so that the
// compiler does not wait for it before unrelated LDS reads; wait_vm0() before the barrier
// that publishes the tile. M0 holds the LDS base (nothing else in these kernels uses M0).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void g2lds16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gsrc) : "m0");
}
// The same load with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset.
__device__ __forceinline__ void g2lds16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase) : "m0");
}
// 4 bytes per lane: lane l's dword lands at lds_base + 4 l.
__device__ __forceinline__ void g2lds4(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(gsrc) : "m0");
}
#pragma clang diagnostic pop

// Waits until at most N vector-memory loads of this wave are outstanding (they complete in
// issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Loads NR rows x CPR chunks into a swizzled tile with all 4 waves of the workgroup.
// src(row, chunk) returns the global address of logical chunk `chunk` of tile row `row`
// (callers clamp rows past the end of the data to a valid row).
template <int CPR, int NR, class Src>
__device__ __forceinline__ void tile_load(bf16* tile, Src src) {
  constexpr int NCH = NR * CPR;           // 16-byte chunks
  constexpr int PERW = NCH / 64 / 4;      // wave-wide loads per wave
  static_assert(NCH % 256 == 0, "tile must split evenly over 4 waves");
  const int w = wave_id(), lane = lane_id();
  const uint32_t base = lds_addr(tile);
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int blk = w * PERW + x;
    const int pch = blk * 64 + lane;      // physical chunk written by this lane
    const int row = pch / CPR;
    const int c = (pch % CPR) ^ swz<CPR>(row);
    g2lds16(src(row, c), base + blk * 1024);
  }
}

// Transposed operand reads. An MFMA operand (8 bf16) whose row index runs along the
// tile's columns: lane l receives tile[row0 + 8 (l / 32) + e][col0 + l % 32] for e = 0..7,
// read with two ds_read_b64_tr_b16. Within each 16-lane group, the transposing read hands
// lane i the (i mod 4)-th element of the 8 bytes addressed by lane 4k + i/4 into slot k, so
// each lane addresses 4 consecutive columns of row row0 + 8 (l / 32) + (l / 4) % 4 (+4 for
// e = 4..7).
//
// The swizzle depends on row & 15 only, so for row0 a multiple of 16 the address is a
// per-lane offset (for row0 = 0; tr_off) plus the constant row0 * row bytes, which the
// reads take as an immediate. Callers compute tr_off once per column block.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int CPR>
__device__ __forceinline__ uint32_t tr_off(int col0, int half, int lane) {
  const int row = 8 * (lane >> 5) + ((lane >> 2) & 3) + 4 * half;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return 2u * (uint32_t)tile_off<CPR>(row, col);
}

// tile: LDS tile base; row0: multiple of 16; off_lo / off_hi: tr_off(col0, 0 / 1, lane)
template <int CPR>
__device__ __forceinline__ bf16x8 lds_tr(const bf16* tile, int row0, uint32_t off_lo, uint32_t off_hi) {
  const char* base = reinterpret_cast<const char*>(tile) + row0 * (CPR * 16);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_lo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off_hi));
  u32x4 r;
  r[0] = __builtin_bit_cast(u32x2, lo)[0];
  r[1] = __builtin_bit_cast(u32x2, lo)[1];
  r[2] = __builtin_bit_cast(u32x2, hi)[0];
  r[3] = __builtin_bit_cast(u32x2, hi)[1];
  return __builtin_bit_cast(bf16x8, r);
}

// Row operand reads: lane l receives tile[row][8 chunk .. 8 chunk + 7] (one ds_read_b128).
// For rows row0 + r with r < 16... the swizzle again depends on the row's low 4 bits only:
// row_off(r, chunk) is the per-lane offset for row0 = 0, and row0 (a multiple of 16) adds a
// constant.
template <int CPR>
__device__ __forceinline__ uint32_t row_off(int row, int chunk) {
  return 16u * (uint32_t)(row * CPR + (chunk ^ swz<CPR>(row)));
}

template <int CPR>
__device__ __forceinline__ bf16x8 lds_row(const bf16* tile, int row0, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + row0 * (CPR * 16) + off);
}

// Runs mma(x, operand) for x = 0..N-1 with the LDS read of operand x issued two products
// ahead (three rotating registers), so each MFMA waits for an operand that was requested
// while the previous ones executed rather than for a read issued just before it.
template <int N, class Read, class Mma>
__device__ __forceinline__ void pipelined(Read read, Mma mma) {
  bf16x8 buf[3];
  buf[0] = read(0);
  if constexpr (N > 1) buf[1] = read(1);
#pragma unroll
  for (int x = 0; x < N; ++x) {
    if (x + 2 < N) buf[(x + 2) % 3] = read(x + 2);
    mma(x, buf[x % 3]);
  }
}

// Marks a register value loaded from global memory before a pipelined loop as settled. The
// compiler's count of outstanding vector-memory loads does not include the loads issued from
// inline assembly (g2lds16 and friends), so at each step's first use of such a value it
// would insert "s_waitcnt vmcnt(N)" for the value's own load, which in hardware waits for the
// youngest N loads in flight: the next steps' tile loads. An empty asm that rewrites the
// value moves that wait to where it stands (the compiler retires the load before the rewrite)
// and leaves the loop free of it. Call it only after a hardware wait that has retired the
// load (run_pipeline's prologue wait does, for loads issued before the pipeline starts).
template <class T>
__device__ __forceinline__ void settle(T& x) {
  asm volatile("" : "+v"(x));
}

// Multi-stage LDS pipeline over the steps 0 .. n_steps - 1 of a work item. Step st
// computes on stage st % NS; the loads of step st + PD (L vector-memory loads per wave and
// step, direct to LDS) are issued at step st and waited for PD - 1 steps later, one barrier
// per step. PD <= NS - 1; with PD < NS - 1 the stages of steps st - 1 .. st + PD - NS stay
// intact during step st (for consumers that lag behind). Steps past n_steps are loaded too
// (callers clamp their rows or read sentinels), so every step issues the same L loads. The
// first NPEEL steps (a multiple of NS) run with `peeled` set, in a loop of their own.
// load(step, stage) and compute(step, stage, peeled) are called with compile-time stage
// indices; settle() runs once after the prologue's wait (see settle above) for the values the
// caller loaded into registers before the pipeline. Leaves no load outstanding.
template <int NS, int PD, int L, int NPEEL, class Load, class Compute, class Settle>
__device__ __forceinline__ void run_pipeline(int n_steps, Load load, Compute compute, Settle settle_regs) {
  static_assert(NS >= 2 && PD >= 1 && PD <= NS - 1 && NPEEL % NS == 0, "pipeline shape");
#pragma unroll
  for (int s = 0; s < PD; ++s) load(s, s);
  wait_vm<L * (PD - 1)>();
  settle_regs();
  __syncthreads();
  auto step = [&](int st, int u, bool peeled) {
    load(st + PD, (u + PD) % NS);
    compute(st, u, peeled);
    wait_vm<L * (PD - 1)>();
    __syncthreads();
  };
  if constexpr (NPEEL > 0) {
    bool more = true;
    for (int st = 0; more && st < NPEEL; st += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        if (st + u >= n_steps) {
          more = false;
          break;
        }
        step(st + u, u, true);
      }
    }
  }
  for (int st = NPEEL; st < n_steps; st += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (st + u < n_steps) step(st + u, u, false);
  }
  wait_vm0();
}

template <int NS, int PD, int L, int NPEEL, class Load, class Compute>
__device__ __forceinline__ void run_pipeline(int n_steps, Load load, Compute compute) {
  run_pipeline<NS, PD, L, NPEEL>(n_steps, load, compute, [] {});
}

// Loads rows j0 .. j0 + NR - 1 (rows past T - 1 re-read row T - 1) of a row-major
// [T, 8 CPR] bf16 matrix into a tile swizzled with swz<CPR>, using all NW waves: wave w
// fills 1 KiB blocks w PERW .. w PERW + PERW - 1. One load per block and lane; the base row
// jb <= every row read keeps the unsigned per-lane offsets non-negative.
template <int CPR, int NR, int NW>
__device__ __forceinline__ void tile_load_rows(bf16* tile, const bf16* src, int j0, int T) {
  constexpr int PERW = NR * CPR / (64 * NW);
  static_assert(PERW >= 1 && NR * CPR == PERW * 64 * NW, "tile must split evenly over the waves");
  const int w = wave_id(), lane = lane_id();
  const int jb = min(j0, T - 1);
  const bf16* base = src + (size_t)jb * (CPR * 8);
#pragma unroll
  for (int x = 0; x < PERW; ++x) {
    const int pch = (w * PERW + x) * 64 + lane, row = pch / CPR;
    const int c = (pch % CPR) ^ swz<CPR>(row);
    const uint32_t o = 2u * (uint32_t)((min(j0 + row, T - 1) - jb) * (CPR * 8) + c * 8);
    g2lds16_s(base, o, lds_addr(tile) + (uint32_t)(w * PERW + x) * 1024u);
  }
}

// tile_load_rows with the per-lane offsets computed once: for a tile whose rows all lie before
// T (every tile of a loop but possibly the one holding the last row), lane l's offset from the
// tile's first row depends on the lane and the wave only, so each load is a scalar base plus
// that offset and costs no vector instruction. Tiles that reach past T take tile_load_rows.
template <int CPR, int NR, int NW>
struct RowTileLoader {
  static constexpr int PERW = NR * CPR / (64 * NW);
  static_assert(PERW >= 1 && NR * CPR == PERW * 64 * NW, "tile must split evenly over the waves");
  uint32_t off[PERW];
  __device__ __forceinline__ RowTileLoader() {
    const int w = wave_id(), lane = lane_id();
#pragma unroll
    for (int x = 0; x < PERW; ++x) {
      const int pch = (w * PERW + x) * 64 + lane, row = pch / CPR;
      const int c = (pch % CPR) ^ swz<CPR>(row);
      off[x] = 2u * (uint32_t)(row * (CPR * 8) + c * 8);
    }
  }
  // rows j0 .. j0 + NR - 1 of the row-major [T, 8 CPR] matrix src
  __device__ __forceinline__ void load(bf16* tile, const bf16* src, int j0, int T) const {
    if (j0 + NR <= T) {
      const bf16* base = src + (size_t)j0 * (CPR * 8);
      const uint32_t lb = lds_addr(tile) + (uint32_t)(wave_id() * PERW) * 1024u;
#pragma unroll
      for (int x = 0; x < PERW; ++x) g2lds16_s(base, off[x], lb + (uint32_t)x * 1024u);
    } else {
      tile_load_rows<CPR, NR, NW>(tile, src, j0, T);
    }
  }
};

// XCD-aware work-item map. MI355X has 8 XCDs, each with its own L2, and workgroup b runs on
// XCD b % 8. Items come in rows (one row per tile position, heaviest row first) of nd
// "stream" items (one per ordinary (b, h): the items of one stream read the same K/V or Q/dO
// rows) followed by nf other items. A row is padded to a multiple of 8 slots, so stream item
// x of every row lands on XCD x % 8 and its reads are shared through one L2; the nf items and
// the empty slots of the padding rotate by row so that every XCD gets the same share of them.
// Returns false for an empty slot; else the row and the item index in the row (0 .. nd + nf).
constexpr int kNumXcd = 8;
__host__ __device__ __forceinline__ int xcd_row_slots(int nd, int nf) {
  return (nd + nf + kNumXcd - 1) / kNumXcd * kNumXcd;
}
__device__ __forceinline__ bool xcd_item(int b, int nd, int nf, int& row, int& item) {
  const int slots = xcd_row_slots(nd, nf);
  row = b / slots;
  const int slot = b % slots;
  if (slot < nd) {
    item = slot;
    return true;
  }
  const int tail = slots - nd;   // nf items and slots - nd - nf empty slots, rotated by row
  const int t = (slot - nd + row * (tail - nf)) % tail;
  item = nd + t;
  return t < nf;
}

// Sum of N values as a balanced tree: a handful of dependent steps instead of an N-long chain.
template <int N>
__device__ __forceinline__ float tree_sum(const float* x) {
  static_assert(N >= 1 && (N & (N - 1)) == 0, "power of two");
  float v[N];
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = x[r];
#pragma unroll
  for (int w = N / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int r = 0; r < w; ++r) v[r] += v[r + w];
  return v[0];
}

// Combine a value across the two half-waves (lanes l and l ^ 32) with v_permlane32_swap (no
// LDS round trip). Swapping two copies of x leaves the lower half's values in the first and
// the upper half's in the second, on every lane. Inline assembly keeps the two copies in
// separate registers (the compiler folds the builtin's results when both inputs are equal).
__device__ __forceinline__ void xhalf_swap(float x, float& lo, float& hi) {
  lo = x;
  hi = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ float xhalf_max(float x) {
  float lo, hi;
  xhalf_swap(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  float lo, hi;
  xhalf_swap(x, lo, hi);
  return lo + hi;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16 a = (bf16)lo, b = (bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)x[e];
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Transposes a 4 (rows) x 8 (columns) block of 16-bit values held as four 16-byte row
// vectors into eight 8-byte column vectors: out[c] = {row0[c], row1[c], row2[c], row3[c]}.
__device__ __forceinline__ void transpose_4x8(const u32x4 (&in)[4], u32x2 (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t a0 = in[0][w], a1 = in[1][w], a2 = in[2][w], a3 = in[3][w];
    out[2 * w][0] = (a0 & 0xffffu) | (a1 << 16);
    out[2 * w][1] = (a2 & 0xffffu) | (a3 << 16);
    out[2 * w + 1][0] = (a0 >> 16) | (a1 & 0xffff0000u);
    out[2 * w + 1][1] = (a2 >> 16) | (a3 & 0xffff0000u);
  }
}

}  // namespace saf
