// rope_qk.hip -- fused per-head RMSNorm + channel-split 3D rotary embedding,
// and the per-head RMSNorm alone.
//
// What it computes (FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder
// with Transformers, Sec. 3.2 "Base Architecture": RMSNorm, and 3D-RoPE
// applied separately to the temporal and spatial axes): for every token and
// head of q and k, y = x / sqrt(mean(x^2) + eps) * g, then each adjacent
// channel pair is rotated by pos_axis * theta^(-j / P_axis).  The norm can be
// left out for q alone (KV-norm, where the same section normalises keys and
// values inside attention) or for both; rms_norm_kernel normalises the values.
//
// Design (HBM-bound, one pass): a workgroup owns a few consecutive tokens.
// It first computes cos/sin for each (token, pair) once -- the angle is
// formed and reduced modulo 2*pi in float64 so large temporal offsets keep
// float32 accuracy, then its sine and cosine are taken in float32 -- into
// LDS, and every q and k head of those tokens reuses them.  Each lane then owns 8 channels (one 16-byte bf16 vector) of
// one head row; the row's sum of squares is reduced across the D/8 lanes of
// the row with cross-lane shuffles.  Loads and stores are 16-byte vectors
// over contiguous memory, so each token's q (and k) block streams through
// once.  In-place operation is safe: a lane reads its 8 channels before it
// writes them.
#include "device_common.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kMaxRopeTok = 32;

template <int D, bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rope_qk_kernel(RopeLaunch p, int tok_per_block) {
  constexpr int P = D / 2;
  constexpr int TPR = D / 8;  // lanes per head row
  __shared__ float2 cs[kMaxRopeTok * P];

  const int64_t rows_total = int64_t(p.B) * p.L;
  const int64_t row0 = int64_t(blockIdx.x) * tok_per_block;
  const int ntok = int(min<int64_t>(tok_per_block, rows_total - row0));
  if (ntok <= 0) return;

  // ---- angles: one (token, pair) per thread iteration ------------------
  const double log2_theta = log2(double(p.theta));
  const int64_t HW = int64_t(p.H) * p.W;
  for (int e = threadIdx.x; e < ntok * P; e += kRopeThreads) {
    const int tl = e / P, pr = e - tl * P;
    const int64_t row = row0 + tl;
    const int64_t i = row % p.L;
    const int64_t n = p.token0 + i;
    int axis, j, Pa;
    if (pr < p.pairs_t) { axis = 0; j = pr; Pa = p.pairs_t; }
    else if (pr < p.pairs_t + p.pairs_h) { axis = 1; j = pr - p.pairs_t; Pa = p.pairs_h; }
    else { axis = 2; j = pr - p.pairs_t - p.pairs_h; Pa = p.pairs_w; }
    int64_t pos;
    if (axis == 0) pos = n / HW + p.t_offset;
    else if (axis == 1) pos = (n / p.W) % p.H;
    else pos = n % p.W;
    const double omega = exp2(-double(j) / double(Pa) * log2_theta);
    double ang = double(pos) * omega;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    // the reduced angle lies in [-pi, pi]: float32 sine and cosine suffice
    float sn, cn;
    sincosf(float(ang), &sn, &cn);
    cs[tl * P + pr] = make_float2(cn, sn);
  }
  __syncthreads();

  const bool has_q = p.q_in != nullptr, has_k = p.k_in != nullptr;
  const int rows_q = has_q ? p.Hq : 0;
  const int rows_per_tok = rows_q + (has_k ? p.Hk : 0);
  const int tasks = ntok * rows_per_tok * TPR;
  const float inv_d = 1.0f / float(D);

  // row index -> (token, row) without an integer division: rt < 2^16, so
  // the float quotient, nudged by half a step, truncates exactly
  const float inv_rpt = 1.0f / float(rows_per_tok);
  for (int t = threadIdx.x; t < tasks; t += kRopeThreads) {
    const int c = t % TPR;
    const int rt = t / TPR;
    const int tl = int((float(rt) + 0.5f) * inv_rpt);
    const int r = rt - tl * rows_per_tok;
    const int64_t row = row0 + tl;
    const bool is_q = r < rows_q;
    const int head = is_q ? r : r - rows_q;
    const int nh = is_q ? p.Hq : p.Hk;
    const int64_t off = (row * nh + head) * int64_t(D) + c * 8;
    const void* src = is_q ? p.q_in : p.k_in;
    void* dst = is_q ? p.q_out : p.k_out;
    const float* gain = is_q ? p.q_gain : p.k_gain;

    float x[8];
    if constexpr (BF16) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
      unpack8(u, x);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    if (is_q ? p.norm_q : p.norm_k) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, TPR);
      const float rinv = 1.0f / sqrtf(fmaf(ss, inv_d, p.eps));
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= rinv;
    }
    if (gain) {
      const float4 ga = *reinterpret_cast<const float4*>(gain + c * 8);
      const float4 gb = *reinterpret_cast<const float4*>(gain + c * 8 + 4);
      x[0] *= ga.x; x[1] *= ga.y; x[2] *= ga.z; x[3] *= ga.w;
      x[4] *= gb.x; x[5] *= gb.y; x[6] *= gb.z; x[7] *= gb.w;
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 a = cs[tl * P + c * 4 + e];
      const float x0 = x[2 * e], x1 = x[2 * e + 1];
      y[2 * e] = x0 * a.x - x1 * a.y;
      y[2 * e + 1] = x0 * a.y + x1 * a.x;
    }
    if constexpr (BF16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + off) = pack8(y);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(dst) + off) = make_float4(y[0], y[1], y[2], y[3]);
      *reinterpret_cast<float4*>(static_cast<float*>(dst) + off + 4) = make_float4(y[4], y[5], y[6], y[7]);
    }
  }
}

// Per-head RMSNorm alone (the values of KV-norm attention): the same lane
// layout as above, D/8 lanes per row, 16-byte loads and stores, in place safe.
template <int D, bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rms_norm_kernel(RmsNormLaunch p) {
  constexpr int TPR = D / 8;
  const int64_t tasks = p.rows * TPR;
  const float inv_d = 1.0f / float(D);
  // tasks and the block size are multiples of TPR, so the lanes of one row
  // enter and leave the loop together and the shuffles stay inside the row
  for (int64_t t = int64_t(blockIdx.x) * kRopeThreads + threadIdx.x; t < tasks;
       t += int64_t(gridDim.x) * kRopeThreads) {
    const int c = int(t % TPR);
    const int64_t off = t * 8;
    float x[8];
    if constexpr (BF16) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.x_in) + off);
      unpack8(u, x);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p.x_in) + off);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p.x_in) + off + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, TPR);
    const float rinv = 1.0f / sqrtf(fmaf(ss, inv_d, p.eps));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= rinv;
    if (p.gain) {
      const float4 ga = *reinterpret_cast<const float4*>(p.gain + c * 8);
      const float4 gb = *reinterpret_cast<const float4*>(p.gain + c * 8 + 4);
      x[0] *= ga.x; x[1] *= ga.y; x[2] *= ga.z; x[3] *= ga.w;
      x[4] *= gb.x; x[5] *= gb.y; x[6] *= gb.z; x[7] *= gb.w;
    }
    if constexpr (BF16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.x_out) + off) = pack8(x);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.x_out) + off) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(static_cast<float*>(p.x_out) + off + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
}

}  // namespace

hipError_t launch_rms_norm(const RmsNormLaunch& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const int64_t tasks = p.rows * (p.D / 8);
  int64_t blocks = (tasks + kRopeThreads - 1) / kRopeThreads;
  if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;  // grid-stride beyond
  dim3 grid(static_cast<unsigned>(blocks));
  if (p.dtype == 0) {
    if (p.D == 128) hipLaunchKernelGGL((rms_norm_kernel<128, true>), grid, dim3(kRopeThreads), 0, s, p);
    else hipLaunchKernelGGL((rms_norm_kernel<64, true>), grid, dim3(kRopeThreads), 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((rms_norm_kernel<128, false>), grid, dim3(kRopeThreads), 0, s, p);
    else hipLaunchKernelGGL((rms_norm_kernel<64, false>), grid, dim3(kRopeThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_rope(const RopeLaunch& p, hipStream_t s) {
  const int64_t rows = int64_t(p.B) * p.L;
  if (rows == 0 || (!p.q_in && !p.k_in)) return hipSuccess;
  const int rows_per_tok = (p.q_in ? p.Hq : 0) + (p.k_in ? p.Hk : 0);
  const int tasks_per_tok = rows_per_tok * (p.D / 8);
  // about 1536 row pieces per workgroup, but at least ~4 workgroups per CU
  // when the call is small: each thread's pieces are loaded one after the
  // other, so a small call needs the parallelism to hide the load latency
  int tok = (1536 + tasks_per_tok - 1) / tasks_per_tok;
  const int64_t min_blocks = 4 * int64_t(device_cus());
  if (rows / tok < min_blocks) tok = int(rows / min_blocks);
  if (tok < 1) tok = 1;
  if (tok > kMaxRopeTok) tok = kMaxRopeTok;
  const int64_t blocks = (rows + tok - 1) / tok;
  dim3 grid(static_cast<unsigned>(blocks));
  if (p.dtype == 0) {
    if (p.D == 128) hipLaunchKernelGGL((rope_qk_kernel<128, true>), grid, dim3(kRopeThreads), 0, s, p, tok);
    else hipLaunchKernelGGL((rope_qk_kernel<64, true>), grid, dim3(kRopeThreads), 0, s, p, tok);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((rope_qk_kernel<128, false>), grid, dim3(kRopeThreads), 0, s, p, tok);
    else hipLaunchKernelGGL((rope_qk_kernel<64, false>), grid, dim3(kRopeThreads), 0, s, p, tok);
  }
  return hipGetLastError();
}

}  // namespace vdit
