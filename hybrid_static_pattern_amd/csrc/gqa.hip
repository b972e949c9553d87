// Gradients of shared key/value heads (grouped-query attention: the GQA path of part 二.4
// of the web page "When Can Attention Heads Be Statically Defined?: 中文精读笔记", section 3.3 /
// Appendix D.2). Query head h reads K and V of head g = h / G, so the gradient of that K or V
// is the sum over the G query heads of its group: dK sums the ordinary heads (a frozen head
// has no query and contributes nothing to dK), dV sums all of them. The backward kernels
// write one dK and dV per query head; this pass adds each group's G slices.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {

namespace {

struct GqaParams {
  const float4* dk_h;   // [B, H, T, D] per query head
  const float4* dv_h;
  float4* dk;           // [B, Hkv, T, D]
  float4* dv;
  int B, H, Hkv, G;
  int row4;             // T * D / 4
  uint8_t frozen[kMaxHeads];
};

// grid (ceil(row4 / 256), Hkv); each thread sums one float4 of every batch entry
__global__ __launch_bounds__(256) void gqa_reduce_kernel(const GqaParams p) {
  const int x = blockIdx.x * 256 + threadIdx.x, g = blockIdx.y;
  if (x >= p.row4) return;
  bool any_dyn = false;
  for (int u = 0; u < p.G; ++u) any_dyn |= p.frozen[g * p.G + u] == 0;
  for (int b = 0; b < p.B; ++b) {
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int u = 0; u < p.G; ++u) {
      const int h = g * p.G + u;
      const size_t src = ((size_t)b * p.H + h) * p.row4 + x;
      const float4 v = p.dv_h[src];
      sv.x += v.x; sv.y += v.y; sv.z += v.z; sv.w += v.w;
      if (!p.frozen[h]) {
        const float4 k = p.dk_h[src];
        sk.x += k.x; sk.y += k.y; sk.z += k.z; sk.w += k.w;
      }
    }
    const size_t dst = ((size_t)b * p.Hkv + g) * p.row4 + x;
    p.dv[dst] = sv;
    if (any_dyn) p.dk[dst] = sk;
  }
}

}  // namespace

hipError_t launch_gqa_reduce(const AttnArgs& a, const float* dk_heads, const float* dv_heads, float* dk,
                             float* dv, hipStream_t s) {
  GqaParams p{};
  p.dk_h = reinterpret_cast<const float4*>(dk_heads);
  p.dv_h = reinterpret_cast<const float4*>(dv_heads);
  p.dk = reinterpret_cast<float4*>(dk);
  p.dv = reinterpret_cast<float4*>(dv);
  p.B = a.B;
  p.H = a.H;
  p.Hkv = a.Hkv;
  p.G = a.G;
  p.row4 = a.T * a.D / 4;
  for (int x = 0; x < a.heads.n_frz; ++x) p.frozen[a.heads.frz[x]] = 1;
  prof_begin("gqa_reduce", s);
  hipLaunchKernelGGL(gqa_reduce_kernel, dim3((p.row4 + 255) / 256, a.Hkv), dim3(256), 0, s, p);
  prof_end(s);
  return hipGetLastError();
}

}  // namespace saf
