// lse_merge.hip -- combine two attention partials over disjoint key sets.
//
// L = ln(e^{L_a} + e^{L_b}), O = e^{L_a - L} O_a + e^{L_b - L} O_b: the
// online-softmax combination that ring attention applies to the partial
// results of successive key/value chunks (ReGenVC: End-to-End Real-Time
// Generative Video Coding at Ultra-Low Bitrate, unified sequence
// parallelism paragraph).  A partial with L = -inf has weight 0.
//
// Elementwise and HBM-bound: each lane owns 8 channels of one (b, l, h) row;
// the D/8 lanes of a row read the two LSE values, form the weights, and
// stream 16-byte (bf16) or 32-byte (float32) vectors.  All reads of a row
// happen before its writes within one wavefront, so o_out may alias o_a.
#include "device_common.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kMergeThreads = 256;

template <bool IN_BF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* x) {
  if constexpr (IN_BF16) {
    unpack8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off), x);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store8(void* base, int64_t off, const float* y) {
  if constexpr (OUT_BF16) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = pack8(y);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off + 4) = make_float4(y[4], y[5], y[6], y[7]);
  }
}

template <int D, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(MergeLaunch p) {
  constexpr int TPR = D / 8;
  const int64_t rows = int64_t(p.B) * p.L * p.H;
  const int64_t gt = int64_t(blockIdx.x) * kMergeThreads + threadIdx.x;
  const int64_t row = gt / TPR;  // (b, l, h) row in [B, L, H] order
  if (row >= rows) return;
  const int c = int(gt % TPR);
  const int h = int(row % p.H);
  const int64_t bl = row / p.H;
  const int64_t l = bl % p.L, b = bl / p.L;
  const int64_t li = (b * p.H + h) * p.L + l;  // [B, H, L]
  const float la = p.lse_a[li], lb = p.lse_b[li];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lo = -INFINITY;
  if (mx != -INFINITY) {
    const float ea = expf(la - mx), eb = expf(lb - mx);
    const float s = ea + eb;
    wa = ea / s;
    wb = eb / s;
    lo = mx + logf(s);
  }
  const int64_t off = row * D + c * 8;
  float xa[8], xb[8], y[8];
  load8<IN_BF16>(p.o_a, off, xa);
  load8<IN_BF16>(p.o_b, off, xb);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = wa * xa[e] + wb * xb[e];
  store8<OUT_BF16>(p.o_out, off, y);
  if (p.lse_out && c == 0) p.lse_out[li] = lo;
}

template <int D>
hipError_t launch_merge_d(const MergeLaunch& p, hipStream_t s) {
  const int64_t threads = int64_t(p.B) * p.L * p.H * (D / 8);
  dim3 grid(static_cast<unsigned>((threads + kMergeThreads - 1) / kMergeThreads));
  const bool ib = p.in_dtype == 0, ob = p.out_dtype == 0;
  if (ib && ob) hipLaunchKernelGGL((lse_merge_kernel<D, true, true>), grid, dim3(kMergeThreads), 0, s, p);
  else if (ib) hipLaunchKernelGGL((lse_merge_kernel<D, true, false>), grid, dim3(kMergeThreads), 0, s, p);
  else if (ob) hipLaunchKernelGGL((lse_merge_kernel<D, false, true>), grid, dim3(kMergeThreads), 0, s, p);
  else hipLaunchKernelGGL((lse_merge_kernel<D, false, false>), grid, dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

// n-way form of the same combination, for the partials of a key-split
// attention call: L = ln sum_s e^{L_s}, O = sum_s e^{L_s - L} O_s.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kMergeThreads) void split_merge_kernel(SplitMergeLaunch p) {
  constexpr int TPR = D / 8;
  const int64_t rows = int64_t(p.B) * p.L * p.H;
  const int64_t gt = int64_t(blockIdx.x) * kMergeThreads + threadIdx.x;
  const int64_t row = gt / TPR;  // (b, l, h) row in [B, L, H] order
  if (row >= rows) return;
  const int c = int(gt % TPR);
  const int h = int(row % p.H);
  const int64_t bl = row / p.H;
  const int64_t l = bl % p.L, b = bl / p.L;
  const int64_t li = (b * p.H + h) * p.L + l;  // [B, H, L]
  const int64_t so = rows * D, sl = rows;      // one whole partial
  float mx = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s) mx = fmaxf(mx, p.part_lse[s * sl + li]);
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lo = -INFINITY;
  if (mx != -INFINITY) {
    float tot = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
      const float w = expf(p.part_lse[s * sl + li] - mx);
      tot += w;
      float x[8];
      load8<false>(p.part_o, s * so + row * D + c * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = fmaf(w, x[e], y[e]);
    }
    const float inv = 1.f / tot;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] *= inv;
    lo = mx + logf(tot);
  }
  store8<OUT_BF16>(p.o, row * D + c * 8, y);
  if (p.lse && c == 0) p.lse[li] = lo;
}

template <int D>
hipError_t launch_split_merge_d(const SplitMergeLaunch& p, hipStream_t s) {
  const int64_t threads = int64_t(p.B) * p.L * p.H * (D / 8);
  dim3 grid(static_cast<unsigned>((threads + kMergeThreads - 1) / kMergeThreads));
  if (p.out_dtype == 0) hipLaunchKernelGGL((split_merge_kernel<D, true>), grid, dim3(kMergeThreads), 0, s, p);
  else hipLaunchKernelGGL((split_merge_kernel<D, false>), grid, dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_merge(const SplitMergeLaunch& p, hipStream_t s) {
  if (int64_t(p.B) * p.L == 0) return hipSuccess;
  return p.D == 128 ? launch_split_merge_d<128>(p, s) : launch_split_merge_d<64>(p, s);
}

hipError_t launch_merge(const MergeLaunch& p, hipStream_t s) {
  if (int64_t(p.B) * p.L == 0) return hipSuccess;
  return p.D == 128 ? launch_merge_d<128>(p, s) : launch_merge_d<64>(p, s);
}

}  // namespace vdit
