// attn_epilogue.hpp -- per-row finishing arithmetic shared by the attention
// kernels: turning a running (max, sum, unnormalised accumulator) into
// (O, LSE), and the log-sum-exp merge of two partials.
#pragma once

#include "device_common.hpp"
#include "vdit_internal.hpp"

namespace vdit {

// Natural-log LSE of a softmax partial whose scores were tracked in log2
// units: m2 = running max of scale*log2(e)*s, l = sum 2^(that - m2).
__device__ __forceinline__ float partial_lse(float m2, float l) {
  return l > 0.f ? m2 * kLn2 + logf(l) : -INFINITY;
}

// Weights of two partials (la, lb natural-log LSEs) in their merge, and the
// merged LSE.  A -inf partial gets weight 0; two -inf partials give 0, 0, -inf.
struct MergeW {
  float wa, wb, lse;
};
__device__ __forceinline__ MergeW merge_weights(float la, float lb) {
  MergeW w;
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) {
    w.wa = 0.f; w.wb = 0.f; w.lse = -INFINITY;
    return w;
  }
  const float ea = expf(la - mx), eb = expf(lb - mx);
  const float s = ea + eb;
  w.wa = ea / s;
  w.wb = eb / s;
  w.lse = mx + logf(s);
  return w;
}

// phi(x) = elu(x) + 1; e^x for x <= 0 as 2^(x log2 e) on the hardware exp2
// (relative error below 1e-6 for |x| < 16, far under the bf16 rounding the
// map's values go through)
__device__ __forceinline__ float phi_elu1(float x) {
  return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * kLog2e);
}

// The linear term's feature map: elu + 1, or the map's cubic (Horner form).
template <bool POLY>
__device__ __forceinline__ float feature_t(float x, const FeatureMap& f) {
  if constexpr (POLY) return fmaf(fmaf(fmaf(f.c[3], x, f.c[2]), x, f.c[1]), x, f.c[0]);
  else return phi_elu1(x);
}
__device__ __forceinline__ float feature(float x, const FeatureMap& f) {
  return f.poly ? feature_t<true>(x, f) : feature_t<false>(x, f);
}

}  // namespace vdit
