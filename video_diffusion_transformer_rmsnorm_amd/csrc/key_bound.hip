// key_bound.hip -- largest squared key norm per (batch, kv head).
//
// Feeds the bounded-score softmax of the attention kernel: by the
// Cauchy-Schwarz inequality a score q . k never exceeds |q| max_j |k_j|, so
// that product bounds a query's row maximum without looking at its scores.
// One pass over the keys (HBM-bound).  The segment's keys form n_parts runs
// of part_len keys (the chunks of the chunk-hybrid mode; one run
// otherwise); workgroup (run r, b, hk, i) reduces keys [i * per, (i + 1) *
// per) of run r; D/8 lanes share one key row (8 bf16 per lane, 16-byte
// loads), their partial sums of squares meet by lane shuffles, and the
// workgroup maximum is written to out[((r * B + b) * Hk + hk) *
// kKeyBoundBlocks + i].
#include "device_common.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

// NT threads per workgroup: 1024 (more loads in flight per CU) when each
// workgroup has at least 192 keys to reduce (64 workgroups per run), else
// 256.
template <int D, int NT>
__global__ __launch_bounds__(NT) void key_bound_kernel(KvSeg seg, int32_t B, int32_t Hk, int64_t part_len, float* out) {
  constexpr int TPR = D / 8;                  // lanes per key row
  constexpr int RPP = NT / TPR;               // rows per pass
  const int i = blockIdx.x % kKeyBoundBlocks;
  const int64_t rbh = blockIdx.x / kKeyBoundBlocks;  // (r * B + b) * Hk + hk
  const int hk = int(rbh % Hk);
  const int64_t b = (rbh / Hk) % B, r = rbh / (int64_t(Hk) * B);
  const int64_t r0 = r * part_len, rlen = min(part_len, seg.len - r0);
  const int64_t per = (rlen + kKeyBoundBlocks - 1) / kKeyBoundBlocks;
  const int64_t j0 = r0 + i * per, j1 = min(r0 + rlen, j0 + per);
  const int tid = threadIdx.x;
  const int c = tid % TPR;
  const uint16_t* base = static_cast<const uint16_t*>(seg.k) + b * seg.bstride + int64_t(hk) * D + c * 8;
  float best = 0.f;
#pragma unroll 4
  for (int64_t j = j0 + tid / TPR; j < j1; j += RPP) {
    float x[8];
    unpack8(*reinterpret_cast<const uint4*>(base + j * int64_t(Hk) * D), x);
    float s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s2 = fmaf(x[e], x[e], s2);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) s2 += __shfl_xor(s2, o);
    best = fmaxf(best, s2);
  }
#pragma unroll
  for (int o = TPR; o < 64; o <<= 1) best = fmaxf(best, __shfl_xor(best, o));
  __shared__ float wmax[NT / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    float m = wmax[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = fmaxf(m, wmax[w]);
    out[rbh * kKeyBoundBlocks + i] = m;
  }
}

}  // namespace

hipError_t launch_key_bound(const KvSeg& seg, int32_t B, int32_t Hk, int32_t D, int64_t part_len, float* out,
                            hipStream_t s) {
  if (part_len <= 0) part_len = seg.len;
  const int64_t parts = part_len > 0 ? (seg.len + part_len - 1) / part_len : 0;
  const int64_t nblk = parts * B * Hk * kKeyBoundBlocks;
  if (nblk == 0) return hipSuccess;
  const bool wide = part_len / kKeyBoundBlocks >= 192;
  const dim3 grid(static_cast<unsigned>(nblk));
  if (D == 128) {
    if (wide) hipLaunchKernelGGL((key_bound_kernel<128, 1024>), grid, dim3(1024), 0, s, seg, B, Hk, part_len, out);
    else hipLaunchKernelGGL((key_bound_kernel<128, 256>), grid, dim3(256), 0, s, seg, B, Hk, part_len, out);
  } else {
    if (wide) hipLaunchKernelGGL((key_bound_kernel<64, 1024>), grid, dim3(1024), 0, s, seg, B, Hk, part_len, out);
    else hipLaunchKernelGGL((key_bound_kernel<64, 256>), grid, dim3(256), 0, s, seg, B, Hk, part_len, out);
  }
  return hipGetLastError();
}

}  // namespace vdit
