// Frozen heads' upstream gradient in float16 for the frozen-head backward of part 二.4 of
// "When Can Attention Heads Be Statically Defined?: 中文精读笔记" (dV = P^T dO only).
//
// The dK/dV kernel forms the frozen product P^T dO with one fp16 MFMA per tile: P in [0, 1]
// keeps 11 significant bits in fp16 (the bf16 sink column of dV, |dV| ~ 17, would keep only 8),
// and dO, which arrives in bf16, converts to fp16 exactly once it lies in fp16's normal range.
// Two passes bring it there. For each batch entry b and frozen head f the slice dO[b, frz[f]]
// (T x D values) is scaled by 2^-e_bf, with e_bf chosen so that the largest magnitude lands in
// [2^14, 2^15): a power of two changes no significant bit, so every value within 2^28 of the
// slice's largest converts exactly, and the dK/dV kernel multiplies its dV columns of batch b
// by 2^e_bf when it stores them.
//   frz_amax_kernel  per (slice, 8192-value block): the block's largest magnitude (the dQ
//                    kernel takes these blocks as extra items when it runs);
//   frz_half_kernel  per (slice, block): the slice's largest magnitude from the block maxima,
//                    e_bf (block 0 writes it), and the block's values scaled and rounded to fp16.
// A slice whose largest magnitude is 0 or not finite keeps e_bf = 0 (infinities and NaN pass
// through to dV as they would in any product).
#include "frz_amax.h"

namespace saf {

namespace {

struct HalfParams {
  FrzAmaxArgs a;
  uint16_t* dh;         // fp16 [B, n_frz, T, D]
  int32_t* dexp;        // [B * n_frz] e_bf
  uint8_t frz[kMaxHeads];
};

__global__ __launch_bounds__(kFrzThreads) void frz_amax_kernel(const HalfParams p) {
  __shared__ float red[kFrzThreads / 64];
  frz_amax_item(p.a, p.frz, blockIdx.x, red);
}

// one-dimensional grid: workgroup x converts block x % nblk of slice x / nblk
__global__ __launch_bounds__(kFrzThreads) void frz_half_kernel(const HalfParams p) {
  __shared__ float red[kFrzThreads / 64];
  const FrzAmaxArgs& a = p.a;
  const int s = blockIdx.x / a.nblk, blk = blockIdx.x % a.nblk;
  const uint16_t* src = a.dO + ((size_t)(s / a.n_frz) * a.H + p.frz[s % a.n_frz]) * a.slice;
  const size_t lo = (size_t)blk * kFrzBlock, hi = min(lo + kFrzBlock, a.slice);
  u32x4 v[kFrzPer];
#pragma unroll
  for (int y = 0; y < kFrzPer; ++y) {
    const size_t x = lo + 8 * (threadIdx.x + (size_t)y * kFrzThreads);
    v[y] = x < hi ? *reinterpret_cast<const u32x4*>(src + x) : u32x4{0u, 0u, 0u, 0u};
  }
  float m = 0.f;
  for (int x = threadIdx.x; x < a.nblk; x += kFrzThreads) m = fmaxf(m, a.amax[(size_t)s * a.nblk + x]);
  m = frz_block_max(m, red);
  // e: the largest magnitude times 2^-e lies in [2^14, 2^15)
  const int e = (m > 0.f && m <= 3.402823466e38f) ? ilogbf(m) - 14 : 0;
  if (blk == 0 && threadIdx.x == 0) p.dexp[s] = e;
  uint16_t* dst = p.dh + (size_t)s * a.slice;
#pragma unroll
  for (int y = 0; y < kFrzPer; ++y) {
    const size_t x = lo + 8 * (threadIdx.x + (size_t)y * kFrzThreads);
    if (x >= hi) continue;
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const _Float16 lo16 = (_Float16)ldexpf(bf16_to_f32(v[y][k] & 0xffffu), -e);
      const _Float16 hi16 = (_Float16)ldexpf(bf16_to_f32(v[y][k] >> 16), -e);
      o[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo16) | ((uint32_t)__builtin_bit_cast(uint16_t, hi16) << 16);
    }
    *reinterpret_cast<u32x4*>(dst + x) = o;
  }
}

HalfParams half_params(const AttnArgs& a, const void* dO, const FrzHalfWs& ws) {
  HalfParams p{};
  p.a = frz_amax_args(a, dO, ws);
  p.dh = ws.dh;
  p.dexp = ws.dexp;
  for (int x = 0; x < a.heads.n_frz; ++x) p.frz[x] = a.heads.frz[x];
  return p;
}

}  // namespace

FrzAmaxArgs frz_amax_args(const AttnArgs& a, const void* dO, const FrzHalfWs& ws) {
  FrzAmaxArgs r;
  r.dO = static_cast<const uint16_t*>(dO);
  r.amax = ws.amax;
  r.H = a.H;
  r.n_frz = a.heads.n_frz;
  r.nblk = frz_half_blocks(a);
  r.slice = (size_t)a.T * a.D;
  return r;
}

hipError_t launch_frz_half(const AttnArgs& a, const void* dO, const FrzHalfWs& ws, bool amax_done, hipStream_t s) {
  if (a.heads.n_frz == 0) return hipSuccess;
  const HalfParams p = half_params(a, dO, ws);
  const dim3 grid(p.a.nblk * a.B * a.heads.n_frz);
  if (!amax_done) {
    prof_begin("frz_amax", s);
    hipLaunchKernelGGL(frz_amax_kernel, grid, dim3(kFrzThreads), 0, s, p);
    prof_end(s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  prof_begin("frz_half", s);
  hipLaunchKernelGGL(frz_half_kernel, grid, dim3(kFrzThreads), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
