// Block maxima of the frozen heads' upstream gradient, the first of the two passes that bring
// it to fp16 (frz_half.hip); shared by its own kernel and the dQ kernel, which takes these
// blocks as extra work items after its own.
#pragma once
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

constexpr int kFrzThreads = 256;
constexpr int kFrzPer = kFrzBlock / (8 * kFrzThreads);   // 16-byte loads per thread and block
static_assert(kFrzPer * 8 * kFrzThreads == kFrzBlock, "block split");

struct FrzAmaxArgs {
  const uint16_t* dO;   // bf16 [B, H, T, D]
  float* amax;          // [B * n_frz, nblk]
  int H, n_frz, nblk;
  size_t slice;         // T * D values
};

// Largest magnitude over the workgroup (256 threads); red: 4 floats of LDS.
__device__ __forceinline__ float frz_block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Item x (0 .. B n_frz nblk - 1): block x % nblk of slice x / nblk, i.e. values
// [blk kFrzBlock, min((blk + 1) kFrzBlock, slice)) of dO[b, frz[f]], b = slice / n_frz,
// f = slice % n_frz; its largest magnitude goes to amax[x]. All 256 threads of the workgroup
// call it; loads are issued before their values are used.
__device__ __forceinline__ void frz_amax_item(const FrzAmaxArgs& a, const uint8_t* frz, int x, float* red) {
  const int s = x / a.nblk, blk = x % a.nblk;
  const uint16_t* src = a.dO + ((size_t)(s / a.n_frz) * a.H + frz[s % a.n_frz]) * a.slice;
  const size_t lo = (size_t)blk * kFrzBlock, hi = min(lo + kFrzBlock, a.slice);
  u32x4 v[kFrzPer];
#pragma unroll
  for (int y = 0; y < kFrzPer; ++y) {
    const size_t e = lo + 8 * (threadIdx.x + (size_t)y * kFrzThreads);
    v[y] = e < hi ? *reinterpret_cast<const u32x4*>(src + e) : u32x4{0u, 0u, 0u, 0u};
  }
  float m = 0.f;
#pragma unroll
  for (int y = 0; y < kFrzPer; ++y)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = fmaxf(m, fabsf(bf16_to_f32(v[y][k] & 0xffffu)));
      m = fmaxf(m, fabsf(bf16_to_f32(v[y][k] >> 16)));
    }
  m = frz_block_max(m, red);
  if (threadIdx.x == 0) a.amax[x] = m;
}

}  // namespace saf
