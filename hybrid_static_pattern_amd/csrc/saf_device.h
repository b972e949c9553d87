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
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

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

__device__ __forceinline__ float wave_shfl_xor32(float x) {
  return __shfl_xor(x, 32, 64);
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
