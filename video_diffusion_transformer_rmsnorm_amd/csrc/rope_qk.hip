// rope_qk.hip -- fused per-head RMSNorm + channel-split 3D rotary embedding,
// and the per-head RMSNorm alone.
//
// What it computes (FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder
// with Transformers, Sec. 3.2 "Base Architecture": RMSNorm, and 3D-RoPE
// applied separately to the temporal and spatial axes): for every token and
// head of q and k, y = x / sqrt(mean(x^2) + eps) * g, then each adjacent
// channel pair is rotated by pos_axis * theta^(-j / P_axis).  The norm can be
// left out for q alone (KV-norm, where the same section normalises keys and
// values inside attention) or for both.  The values of the same tokens can
// ride along (vdit_rope_qkv): copied, or normalised without rotation, in the
// same launch; rms_norm_kernel normalises values on their own.
//
// Design (HBM-bound, one pass): a workgroup owns a few consecutive tokens.
// Each thread first requests its first 16-byte piece of q, k or v, then the
// workgroup computes cos/sin for each (token, pair) once -- the angle
// (position times the pair's frequency, a power of a per-axis ratio that the
// host forms in float64) is reduced modulo 2*pi in float64 so large temporal
// offsets keep float32 accuracy, then its sine and cosine are taken in
// float32 -- into LDS, and every q and k head of those tokens reuses them.
// Each lane then owns 8 channels (one 16-byte bf16 vector) of one head row;
// the row's sum of squares is reduced across the D/8 lanes of the row with
// cross-lane shuffles.  Loads and stores are 16-byte vectors over contiguous
// memory, so each token's q, k (and v) blocks stream through once.  In-place
// operation is safe: a lane reads its 8 channels before it writes them.
#include <cmath>

#include "device_common.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kRopeThreads = 256;

// One of three values by a piece's kind (q, k or v), chosen on values: a
// choice between captured references would select their addresses and keep
// the captured locals in scratch memory.
template <class T>
__device__ __forceinline__ T by_kind(bool is_k, bool is_v, T q, T k, T v) {
  return is_v ? v : (is_k ? k : q);
}
constexpr int kMaxRopeTok = 32;

// HAS_V: the instance that also passes values through (vdit_rope_qkv); the
// q/k-only instance carries none of that code.
template <int D, bool BF16, bool HAS_V>
__global__ __launch_bounds__(kRopeThreads) void rope_qk_kernel(RopeLaunch p, int tok_per_block) {
  constexpr int P = D / 2;
  constexpr int TPR = D / 8;  // lanes per head row
  __shared__ float2 cs[kMaxRopeTok * P];

  const int64_t rows_total = int64_t(p.B) * p.L;
  const int64_t row0 = int64_t(blockIdx.x) * tok_per_block;
  const int ntok = int(min<int64_t>(tok_per_block, rows_total - row0));
  if (ntok <= 0) return;

  // (per-lane choices below pick between these values, not between fields
  // of the argument block, which would be a load from a per-lane address)
  const void* const q_in = p.q_in;
  const void* const k_in = p.k_in;
  const void* const v_in = p.v_in;
  void* const q_out = p.q_out;
  void* const k_out = p.k_out;
  void* const v_out = p.v_out;
  const float* const q_gain = p.q_gain;
  const float* const k_gain = p.k_gain;
  const float* const v_gain = p.v_gain;
  const int Hq = p.Hq, Hk = p.Hk;
  const bool norm_q = p.norm_q != 0, norm_k = p.norm_k != 0, norm_v = p.norm_v != 0;
  const bool has_q = q_in != nullptr, has_k = k_in != nullptr, has_v = HAS_V && v_in != nullptr;
  const int rows_q = has_q ? Hq : 0;
  const int rows_qk = rows_q + (has_k ? Hk : 0);
  const int rows_per_tok = rows_qk + (has_v ? Hk : 0);
  const int tasks = ntok * rows_per_tok * TPR;
  const float inv_d = 1.0f / float(D);

  // piece t of the workgroup: 8 channels of one q, k or v head row (a
  // token's rows in that order).  Row index -> (token, row) without an
  // integer division: rt < 2^16, so the float quotient, nudged by half a
  // step, truncates exactly.
  struct Piece {
    int64_t off;
    int tl, c;
    bool is_k, is_v;  // else a q row
  };
  const float inv_rpt = 1.0f / float(rows_per_tok);
  auto locate = [&](int t) {
    Piece pc;
    pc.c = t % TPR;
    const int rt = t / TPR;
    pc.tl = int((float(rt) + 0.5f) * inv_rpt);
    const int r = rt - pc.tl * rows_per_tok;
    pc.is_v = HAS_V && r >= rows_qk;
    pc.is_k = !pc.is_v && r >= rows_q;
    const int head = r - by_kind(pc.is_k, pc.is_v, 0, rows_q, rows_qk);
    const int nh = by_kind(pc.is_k, pc.is_v, Hq, Hk, Hk);
    pc.off = ((row0 + pc.tl) * nh + head) * int64_t(D) + pc.c * 8;
    return pc;
  };
  // the raw 16 (bf16) or 32 (float32) bytes of a piece
  struct Raw {
    uint4 a, b;
  };
  auto load_raw = [&](const Piece& pc) {
    Raw w;
    const void* src = by_kind(pc.is_k, pc.is_v, q_in, k_in, v_in);
    if constexpr (BF16) {
      w.a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + pc.off);
      w.b = make_uint4(0, 0, 0, 0);
    } else {
      w.a = *reinterpret_cast<const uint4*>(static_cast<const float*>(src) + pc.off);
      w.b = *reinterpret_cast<const uint4*>(static_cast<const float*>(src) + pc.off + 4);
    }
    return w;
  };
  // Each thread's first piece is requested before the angles are formed, so
  // the memory latency passes under that arithmetic (its bytes are only
  // looked at after the barrier below); in a workgroup of at most two pieces
  // per thread (a decode frame's one-token workgroups) the second piece goes
  // out with it, so the two latencies overlap.  (Unconditional within the
  // workgroup: a thread past the end reads an in-bounds piece it does not
  // use, so no wait below has to allow for a load that may be missing.)
  const int tf = threadIdx.x, ts = tf + kRopeThreads;
  const bool two = tasks <= 2 * kRopeThreads;  // workgroup-uniform
  const Piece pf = locate(min(tf, tasks - 1));
  const Raw wf = load_raw(pf);
  const Piece ps = locate(min(ts, tasks - 1));
  Raw ws;
  if (two) ws = load_raw(ps);
  const double base_t = p.omega_base[0], base_h = p.omega_base[1], base_w = p.omega_base[2];

  // ---- angles: one (token, pair) per thread iteration ------------------
  const int64_t HW = int64_t(p.H) * p.W;
  for (int e = threadIdx.x; e < ntok * P; e += kRopeThreads) {
    const int tl = e / P, pr = e - tl * P;
    const int64_t row = row0 + tl;
    const int64_t i = row % p.L;
    const int64_t n = p.token0 + i;
    int64_t pos;
    int j;
    double base;
    if (pr < p.pairs_t) { pos = n / HW + p.t_offset; j = pr; base = base_t; }
    else if (pr < p.pairs_t + p.pairs_h) { pos = (n / p.W) % p.H; j = pr - p.pairs_t; base = base_h; }
    else { pos = n % p.W; j = pr - p.pairs_t - p.pairs_h; base = base_w; }
    // frequency theta^(-j / P_axis) = base^j by squaring (j < 64): within
    // ~64 float64 ulps, far below what the float32 sine and cosine resolve
    double om = 1.0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      if ((j >> bit) & 1) om *= base;
      base *= base;
    }
    double ang = double(pos) * om;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    // the reduced angle lies in [-pi, pi]: float32 sine and cosine suffice
    float sn, cn;
    sincosf(float(ang), &sn, &cn);
    cs[tl * P + pr] = make_float2(cn, sn);
  }
  __syncthreads();

  auto process = [&](const Piece& pc, const Raw& w) {
    float x[8];
    if constexpr (BF16) {
      unpack8(w.a, x);
    } else {
      x[0] = __uint_as_float(w.a.x); x[1] = __uint_as_float(w.a.y);
      x[2] = __uint_as_float(w.a.z); x[3] = __uint_as_float(w.a.w);
      x[4] = __uint_as_float(w.b.x); x[5] = __uint_as_float(w.b.y);
      x[6] = __uint_as_float(w.b.z); x[7] = __uint_as_float(w.b.w);
    }
    if (by_kind(pc.is_k, pc.is_v, norm_q, norm_k, norm_v)) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
      for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, TPR);
      const float rinv = 1.0f / sqrtf(fmaf(ss, inv_d, p.eps));
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= rinv;
    }
    const float* gain = by_kind(pc.is_k, pc.is_v, q_gain, k_gain, v_gain);
    if (gain) {
      const float4 ga = *reinterpret_cast<const float4*>(gain + pc.c * 8);
      const float4 gb = *reinterpret_cast<const float4*>(gain + pc.c * 8 + 4);
      x[0] *= ga.x; x[1] *= ga.y; x[2] *= ga.z; x[3] *= ga.w;
      x[4] *= gb.x; x[5] *= gb.y; x[6] *= gb.z; x[7] *= gb.w;
    }
    float y[8];
    if (pc.is_v) {  // values are not rotated
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 a = cs[pc.tl * P + pc.c * 4 + e];
        const float x0 = x[2 * e], x1 = x[2 * e + 1];
        y[2 * e] = x0 * a.x - x1 * a.y;
        y[2 * e + 1] = x0 * a.y + x1 * a.x;
      }
    }
    void* dst = by_kind(pc.is_k, pc.is_v, q_out, k_out, v_out);
    if constexpr (BF16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + pc.off) = pack8(y);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(dst) + pc.off) = make_float4(y[0], y[1], y[2], y[3]);
      *reinterpret_cast<float4*>(static_cast<float*>(dst) + pc.off + 4) = make_float4(y[4], y[5], y[6], y[7]);
    }
  };
  // (tasks and the block size are multiples of TPR, so the lanes of one row
  // take the same iterations and the shuffles stay inside the row)
  if (tf < tasks) process(pf, wf);
  if (two) {
    if (ts < tasks) process(ps, ws);
    return;
  }
  for (int t = ts; t < tasks; t += kRopeThreads) {
    const Piece pc = locate(t);
    process(pc, load_raw(pc));
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
  if (rows == 0 || (!p.q_in && !p.k_in && !p.v_in)) return hipSuccess;
  const int rows_per_tok = (p.q_in ? p.Hq : 0) + (p.k_in ? p.Hk : 0) + (p.v_in ? p.Hk : 0);
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
  // per-axis frequency ratios theta^(-1 / P_axis), in float64, once per call
  RopeLaunch q = p;
  const double log2_theta = std::log2(double(p.theta));
  const int pa[3] = {p.pairs_t, p.pairs_h, p.pairs_w};
  for (int a = 0; a < 3; ++a) q.omega_base[a] = pa[a] > 0 ? std::exp2(-log2_theta / double(pa[a])) : 1.0;
  const bool v = p.v_in != nullptr;
  if (p.dtype == 0) {
    if (p.D == 128) {
      if (v) hipLaunchKernelGGL((rope_qk_kernel<128, true, true>), grid, dim3(kRopeThreads), 0, s, q, tok);
      else hipLaunchKernelGGL((rope_qk_kernel<128, true, false>), grid, dim3(kRopeThreads), 0, s, q, tok);
    } else {
      if (v) hipLaunchKernelGGL((rope_qk_kernel<64, true, true>), grid, dim3(kRopeThreads), 0, s, q, tok);
      else hipLaunchKernelGGL((rope_qk_kernel<64, true, false>), grid, dim3(kRopeThreads), 0, s, q, tok);
    }
  } else {
    if (p.D == 128) {
      if (v) hipLaunchKernelGGL((rope_qk_kernel<128, false, true>), grid, dim3(kRopeThreads), 0, s, q, tok);
      else hipLaunchKernelGGL((rope_qk_kernel<128, false, false>), grid, dim3(kRopeThreads), 0, s, q, tok);
    } else {
      if (v) hipLaunchKernelGGL((rope_qk_kernel<64, false, true>), grid, dim3(kRopeThreads), 0, s, q, tok);
      else hipLaunchKernelGGL((rope_qk_kernel<64, false, false>), grid, dim3(kRopeThreads), 0, s, q, tok);
    }
  }
  return hipGetLastError();
}

}  // namespace vdit
