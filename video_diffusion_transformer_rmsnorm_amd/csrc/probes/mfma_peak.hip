// mfma_peak.hip -- measurement probe: the sustained rate of the bf16 matrix
// cores on this device, as the ceiling the attention kernel is compared
// with (next to the nominal 2.5 PFLOP/s).  Not part of the library's ABI; the
// benchmark loads it from libvdit_probes.so.
//
// Every wavefront keeps four independent 32x32 accumulators and issues
// v_mfma_f32_32x32x16_bf16 back to back from registers (no memory traffic in
// the loop), two wavefronts per SIMD as in the attention kernel.  The clock
// of a power-limited part depends on how much the operands toggle, so the
// operands come from caller-supplied data: with `vary` set each step takes
// the next of eight operand pairs (random data keeps switching the
// multipliers, like attention on real-valued inputs); otherwise one pair is
// reused.  FLOPs = blocks * 4 wavefronts * iters * 8 MFMAs * 32768.
//
// A second probe gives the cost of the exponential the softmax issues per
// score relative to a plain float32 operation: eight independent chains per
// thread of v_exp_f32 (x <- 2^-x, which stays in (0, 1]), of v_sub_f32
// (x <- 1 - x), or of one of each per step, at eight wavefronts per SIMD so
// that the chains' latency is hidden and the time is the VALU issue.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool VARY>
__global__ __launch_bounds__(256, 2) void mfma_peak_kernel(const uint4* seed, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(bf16x8, seed[(2 * j) * 64 + lane]);
    b[j] = __builtin_bit_cast(bf16x8, seed[(2 * j + 1) * 64 + lane]);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int x = VARY ? j : 0;
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], b[x], acc[j & 3], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int KIND>  // 0: exponentials, 1: subtractions, 2: one of each per step
__global__ __launch_bounds__(256) void valu_rate_kernel(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.001f * float(threadIdx.x + j);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (KIND == 0) x[j] = __builtin_amdgcn_exp2f(-x[j]);
      else if constexpr (KIND == 1) x[j] = 1.0f - x[j];
      else x[j] = 1.0f - __builtin_amdgcn_exp2f(-x[j]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// out: blocks * 256 floats on the device.  kind 0: v_exp_f32 chains, 1:
// v_sub_f32 chains, 2: one of each per step; blocks * 4 wavefronts * iters *
// 8 chain steps in all.  Launches on `stream`.
extern "C" int vdit_probe_valu_rate(int kind, float* out, int iters, int blocks, hipStream_t stream) {
  if (!out || iters <= 0 || blocks <= 0 || kind < 0 || kind > 2) return int(hipErrorInvalidValue);
  if (kind == 0) hipLaunchKernelGGL(valu_rate_kernel<0>, dim3(blocks), dim3(256), 0, stream, out, iters);
  else if (kind == 1) hipLaunchKernelGGL(valu_rate_kernel<1>, dim3(blocks), dim3(256), 0, stream, out, iters);
  else hipLaunchKernelGGL(valu_rate_kernel<2>, dim3(blocks), dim3(256), 0, stream, out, iters);
  return int(hipGetLastError());
}

// seed: 16 * 64 uint4 (bf16 operand data) on the device; out: blocks * 256
// floats.  Launches `blocks` workgroups of 4 wavefronts on `stream`.
extern "C" int vdit_probe_mfma_peak(const void* seed, float* out, int iters, int vary, int blocks,
                                    hipStream_t stream) {
  if (!seed || !out || iters <= 0 || blocks <= 0) return int(hipErrorInvalidValue);
  if (vary)
    hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(seed), out, iters);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(seed), out, iters);
  return int(hipGetLastError());
}
