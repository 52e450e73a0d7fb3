// hybrid_state.hip -- running linear-attention state of the chunk-hybrid mode.
//
// MobileWan: Closing the Quality Gap for Mobile Video Diffusion (review of
// Sec. 3.2) runs the hybrid attention as an RNN over chunks whose fixed-size
// state (s_t, z_t) summarises every earlier chunk through causal linear
// attention: s += phi(K_c)^T V_c, z += sum_j phi(k_j) after chunk c, with
// phi = elu + 1.  Chunk c's queries need the state *before* it, S_c.
//
// Instead of a serial loop over chunks this is a two-pass scan:
//  1. delta pass: every (chunk, token split, batch, kv head) workgroup forms
//     its partial dS = phi(K)^T V and dz = sum phi(k) over its tokens in
//     float32 (stored transposed, [d_out][d_in]);
//  2. scan pass: one lane per state element walks the chunks in order,
//     writing S_c (exclusive prefix, starting from the incoming state) and
//     adding the chunk's split deltas; it ends by writing the outgoing state.
//     For bf16 models S_c is written as a bf16 hi + lo pair (the attention
//     kernel consumes it on the matrix cores with ~16 significant bits);
//     for float32 models as float32.
#include "attn_epilogue.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kDeltaThreads = 256;
constexpr int kDeltaBN = 32;  // tokens per LDS tile

template <int D, bool BF16>
__global__ __launch_bounds__(kDeltaThreads) void hybrid_delta_kernel(HybridStateLaunch p) {
  constexpr int NO = D * D / kDeltaThreads;  // outputs per thread
  constexpr int TPR = D / NO;                // threads per d_in row
  __shared__ float kt[kDeltaBN][D];
  __shared__ float vt[kDeltaBN][D];

  // blockIdx.x = ((c * nsplit + s) * B + b) * Hk + hk
  int64_t bid = blockIdx.x;
  const int hk = int(bid % p.Hk); bid /= p.Hk;
  const int b = int(bid % p.B); bid /= p.B;
  const int s = int(bid % p.nsplit);
  const int64_t c = bid / p.nsplit;
  const int64_t c0 = c * p.chunk, c1 = min(p.L, c0 + p.chunk);
  const int64_t per = (c1 - c0 + p.nsplit - 1) / p.nsplit;
  const int64_t t0 = min(c1, c0 + s * per), t1 = min(c1, t0 + per);

  const int tid = threadIdx.x;
  const int din = tid / TPR;
  const int dout0 = (tid % TPR) * NO;
  float acc[NO];
#pragma unroll
  for (int e = 0; e < NO; ++e) acc[e] = 0.f;
  float zacc = 0.f;

  for (int64_t j0 = t0; j0 < t1; j0 += kDeltaBN) {
    const int nv = int(min<int64_t>(kDeltaBN, t1 - j0));
    __syncthreads();
    for (int e = tid; e < kDeltaBN * D; e += kDeltaThreads) {
      const int jj = e / D, d = e % D;
      float kx = 0.f, vx = 0.f;
      if (jj < nv) {
        const int64_t off = ((int64_t(b) * p.L + j0 + jj) * p.Hk + hk) * D + d;
        if constexpr (BF16) {
          kx = phi_elu1(bf16_to_f32(static_cast<const uint16_t*>(p.k)[off]));
          vx = bf16_to_f32(static_cast<const uint16_t*>(p.v)[off]);
        } else {
          kx = phi_elu1(static_cast<const float*>(p.k)[off]);
          vx = static_cast<const float*>(p.v)[off];
        }
      }
      kt[jj][d] = kx;
      vt[jj][d] = vx;
    }
    __syncthreads();
    for (int jj = 0; jj < nv; ++jj) {
      const float fk = kt[jj][din];
      zacc += fk;
#pragma unroll
      for (int e = 0; e < NO; ++e) acc[e] = fmaf(fk, vt[jj][dout0 + e], acc[e]);
    }
  }
  const int64_t slot = ((c * p.nsplit + s) * p.B + b) * p.Hk + hk;
  float* ds = p.ds + slot * D * D;
#pragma unroll
  for (int e = 0; e < NO; ++e) ds[int64_t(dout0 + e) * D + din] = acc[e];
  if (dout0 == 0) p.dz[slot * D + din] = zacc;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void hybrid_scan_kernel(HybridStateLaunch p) {
  constexpr int NE = D * D + D;
  const int64_t gt = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t bh = gt / NE;
  if (bh >= int64_t(p.B) * p.Hk) return;
  const int e = int(gt % NE);
  const bool is_z = e >= D * D;
  const int dout = is_z ? 0 : e / D, din = is_z ? e - D * D : e % D;
  float run = is_z ? p.z_in[bh * D + din] : p.s_in[bh * D * D + int64_t(din) * D + dout];
  const int64_t plane = p.n_chunks * int64_t(p.B) * p.Hk * D * D;
  for (int64_t c = 0; c < p.n_chunks; ++c) {
    const int64_t cs = c * p.B * p.Hk + bh;  // [c][b][hk]
    if (is_z) {
      p.zc[cs * D + din] = run;
    } else if constexpr (BF16) {
      uint16_t* hi = static_cast<uint16_t*>(p.sc) + cs * D * D + e;
      const uint16_t h = f32_to_bf16(run);
      hi[0] = h;
      hi[plane] = f32_to_bf16(run - bf16_to_f32(h));
    } else {
      static_cast<float*>(p.sc)[cs * D * D + e] = run;
    }
    for (int s = 0; s < p.nsplit; ++s) {
      const int64_t slot = (c * p.nsplit + s) * p.B * p.Hk + bh;
      run += is_z ? p.dz[slot * D + din] : p.ds[slot * D * D + e];
    }
  }
  if (is_z) p.z_out[bh * D + din] = run;
  else p.s_out[bh * D * D + int64_t(din) * D + dout] = run;
}

template <int D, bool BF16>
hipError_t launch_d(const HybridStateLaunch& p, hipStream_t s) {
  const int64_t nblk = p.n_chunks * p.nsplit * p.B * p.Hk;
  if (nblk > 0) {
    hipLaunchKernelGGL((hybrid_delta_kernel<D, BF16>), dim3(static_cast<unsigned>(nblk)), dim3(kDeltaThreads), 0, s, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t nthr = int64_t(p.B) * p.Hk * (D * D + D);
  hipLaunchKernelGGL((hybrid_scan_kernel<D, BF16>), dim3(static_cast<unsigned>((nthr + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hybrid_state(const HybridStateLaunch& p, hipStream_t s) {
  if (int64_t(p.B) * p.Hk == 0) return hipSuccess;
  const bool bf = p.dtype == 0;
  if (p.D == 128) return bf ? launch_d<128, true>(p, s) : launch_d<128, false>(p, s);
  return bf ? launch_d<64, true>(p, s) : launch_d<64, false>(p, s);
}

}  // namespace vdit
