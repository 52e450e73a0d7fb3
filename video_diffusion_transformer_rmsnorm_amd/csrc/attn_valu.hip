// attn_valu.hip -- float32 flash attention on the vector ALUs.
//
// Serves VDIT_F32 tensors (the matrix cores have no fast float32 path worth
// the complexity for the small fp32 workloads), in every mode.  Exact
// softmax attention O = softmax(scale Q K^T) V per head (FlashDecoder:
// Real-Time Latent-to-Pixel Streaming Decoder with Transformers, Sec. 3.3
// runs standard exact attention per frame), evaluated as a tiled online
// softmax: one lane per query row, 32-key K/V tiles staged in LDS as
// float32 and read as broadcasts, the running max and sum kept in log2
// units.  The epilogues are the same as in the bf16 matrix-core kernel:
// plain, ring (fold into a float32 running partial with the log-sum-exp
// merge) and chunk-hybrid (joint normalisation with the linear-attention
// partial phi(q)^T S_c / phi(q)^T z_c).
#include "attn_epilogue.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kValuBM = 64;  // queries per workgroup (one wavefront)
constexpr int kValuBN = 32;  // keys per LDS tile

template <bool BF16>
__device__ __forceinline__ float ld(const void* base, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <bool BF16>
__device__ __forceinline__ void st(void* base, int64_t i, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[i] = f32_to_bf16(x);
  else static_cast<float*>(base)[i] = x;
}

template <int D, bool BF16>
__global__ __launch_bounds__(kValuBM) void attn_valu_kernel(AttnLaunch p, int64_t total) {
  __shared__ float ks[kValuBN][D];
  __shared__ float vs[kValuBN][D];

  const int64_t lid = xcd_remap(blockIdx.x, total);
  const int lane = threadIdx.x;
  const bool hybrid = p.epi == kEpiHybrid;
  int64_t q_begin, q_end, chunk_id = 0;
  int h, b;
  KvSeg segs[kMaxSeg];
  int nseg;
  if (!hybrid) {
    const int64_t tiles = (p.Lq + kValuBM - 1) / kValuBM;
    const int64_t qt = lid % tiles, rest = lid / tiles;
    h = int(rest % p.Hq);
    b = int(rest / p.Hq);
    q_begin = qt * kValuBM;
    q_end = min(p.Lq, q_begin + kValuBM);
    nseg = p.nseg;
    for (int s = 0; s < kMaxSeg; ++s) segs[s] = p.seg[s];
  } else {
    const int64_t tpc = (p.chunk + kValuBM - 1) / kValuBM;
    const int64_t t = lid % tpc, rest = lid / tpc;
    chunk_id = rest % p.n_chunks;
    const int64_t rest2 = rest / p.n_chunks;
    h = int(rest2 % p.Hq);
    b = int(rest2 / p.Hq);
    const int64_t c0 = chunk_id * p.chunk;
    const int64_t c1 = min(p.Lq, c0 + p.chunk);
    q_begin = c0 + t * kValuBM;
    q_end = min(c1, q_begin + kValuBM);
    if (q_begin >= q_end) return;
    const int64_t es = BF16 ? 2 : 4;
    // softmax window: the chunk's keys and the hyb_overlap keys before them
    const int64_t w0 = max<int64_t>(0, p.hyb_ctx + c0 - p.hyb_overlap), w1 = p.hyb_ctx + c1;
    nseg = 1;
    segs[0].k = static_cast<const char*>(p.hk) + w0 * p.Hk * D * es;
    segs[0].v = static_cast<const char*>(p.hv) + w0 * p.Hk * D * es;
    segs[0].len = w1 - w0;
    segs[0].bstride = p.hyb_lkv * p.Hk * D;
  }
  const int hk = h / (p.Hq / p.Hk);
  const int64_t qi = q_begin + lane;
  const bool valid = qi < q_end;

  float qv[D];
  {
    const int64_t base = ((int64_t(b) * p.Lq + (valid ? qi : q_begin)) * p.Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] = ld<BF16>(p.q, base + d);
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int s = 0; s < nseg; ++s) {
    const KvSeg sg = segs[s];
    for (int64_t j0 = 0; j0 < sg.len; j0 += kValuBN) {
      const int nv = int(min<int64_t>(kValuBN, sg.len - j0));
      __syncthreads();
      for (int e = lane; e < kValuBN * D; e += kValuBM) {
        const int jj = e / D, d = e % D;
        float kx = 0.f, vx = 0.f;
        if (jj < nv) {
          const int64_t off = int64_t(b) * sg.bstride + ((j0 + jj) * p.Hk + hk) * D + d;
          kx = ld<BF16>(sg.k, off);
          vx = ld<BF16>(sg.v, off);
        }
        ks[jj][d] = kx;
        vs[jj][d] = vx;
      }
      __syncthreads();
      float sc[kValuBN];
      float mt = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < kValuBN; ++jj) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(qv[d], ks[jj][d], dot);
        sc[jj] = jj < nv ? dot * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, sc[jj]);
      }
      const float mn = fmaxf(m, mt);
      const float alpha = exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
      m = mn;
#pragma unroll
      for (int jj = 0; jj < kValuBN; ++jj) {
        const float pj = exp2f(sc[jj] - mn);
        l += pj;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(pj, vs[jj][d], acc[d]);
      }
    }
  }

  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_s = partial_lse(m, l);
  const int64_t orow = ((int64_t(b) * p.Lq + qi) * p.Hq + h) * D;
  const int64_t lrow = (int64_t(b) * p.Hq + h) * p.Lq + qi;

  if (p.epi == kEpiPlain) {
#pragma unroll
    for (int d = 0; d < D; ++d) st<BF16>(p.o, orow + d, acc[d] * inv);
    if (p.lse) p.lse[lrow] = lse_s;
    return;
  }
  if (p.epi == kEpiRing) {
    float lse_out = lse_s, wa = 0.f, wb = 1.f;
    if (p.has_prev) {
      const MergeW w = merge_weights(p.part_lse[lrow], lse_s);
      wa = w.wa; wb = w.wb; lse_out = w.lse;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      float y = wb * acc[d] * inv;
      if (p.has_prev) y = fmaf(wa, p.part_o[orow + d], y);
      if (p.final_out) st<BF16>(p.o, orow + d, y);
      else p.part_o[orow + d] = y;
    }
    if (p.final_out) {
      if (p.lse) p.lse[lrow] = lse_out;
    } else {
      p.part_lse[lrow] = lse_out;
    }
    return;
  }
  // chunk-hybrid: linear partial from the state before this chunk
  const int64_t sidx = (chunk_id * p.B + b) * p.Hk + hk;
  const float* S = static_cast<const float*>(p.st) + sidx * D * D;  // [d_out][d_in]
  const float* z = p.zc + sidx * D;
  float fq[D];
  float den = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    fq[d] = feature(qv[d], p.phi_q);
    den = fmaf(fq[d], z[d], den);
  }
  const float lse_l = den > 0.f ? logf(den) : -INFINITY;
  const MergeW w = merge_weights(lse_s, lse_l);
  const float inv_den = den > 0.f ? 1.f / den : 0.f;
  for (int d = 0; d < D; ++d) {
    float num = 0.f;
    for (int e = 0; e < D; ++e) num = fmaf(fq[e], S[d * D + e], num);
    st<BF16>(p.o, orow + d, w.wa * acc[d] * inv + w.wb * num * inv_den);
  }
  if (p.lse) p.lse[lrow] = w.lse;
}

}  // namespace

hipError_t launch_attn_f32(const AttnLaunch& p, hipStream_t s) {
  int64_t total;
  if (p.epi == kEpiHybrid) {
    const int64_t tpc = (p.chunk + kValuBM - 1) / kValuBM;
    total = tpc * p.n_chunks * p.Hq * p.B;
  } else {
    total = ((p.Lq + kValuBM - 1) / kValuBM) * p.Hq * p.B;
  }
  if (total == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(total));
  if (p.D == 128) hipLaunchKernelGGL((attn_valu_kernel<128, false>), grid, dim3(kValuBM), 0, s, p, total);
  else hipLaunchKernelGGL((attn_valu_kernel<64, false>), grid, dim3(kValuBM), 0, s, p, total);
  return hipGetLastError();
}

}  // namespace vdit
