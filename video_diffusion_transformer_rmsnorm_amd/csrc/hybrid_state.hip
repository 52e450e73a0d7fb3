// hybrid_state.hip -- running linear-attention state of the chunk-hybrid mode.
//
// MobileWan: Closing the Quality Gap for Mobile Video Diffusion (review of
// Sec. 3.2) runs the hybrid attention as an RNN over chunks whose fixed-size
// state (s_t, z_t) summarises every earlier chunk through causal linear
// attention: s += phi(K_c)^T V_c, z += sum_j phi(k_j) after chunk c, with
// phi = elu + 1 or the caller's cubic phi_k.  Chunk c's queries need the
// state *before* it, S_c.  When the softmax windows overlap (the window of
// chunk c starts `overlap` keys before the chunk), S_c covers the keys
// before that window instead, so the delta of chunk c runs from the start
// of its window to the start of the next one (hybrid_delta_range) and the
// outgoing state leaves out the last `overlap` keys, which the next call
// receives as context.
//
// Instead of a serial loop over chunks this is a two-pass scan:
//  1. delta pass: every (chunk, token split, batch, kv head) workgroup forms
//     its partial dS = phi(K)^T V and dz = sum phi(k) over its tokens in
//     float32 (stored transposed, [d_out][d_in]);
//  2. scan pass: one lane per state element walks the chunks in order,
//     writing S_c (exclusive prefix, starting from the incoming state) and
//     adding the chunk's split deltas; it ends by writing the outgoing state.
//     For bf16 models S_c is written in bf16 (the operand of the attention
//     kernel's matrix-core epilogue, next to phi(q) in bf16; the running
//     state itself stays float32); for float32 models as float32.
#include "attn_epilogue.hpp"
#include "device_common.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kDeltaThreads = 256;
constexpr int kDeltaBN = 32;  // tokens per LDS tile

template <int D, bool BF16, bool POLY>
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
  int64_t c0, c1;
  hybrid_delta_range(p, c, &c0, &c1);
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
        const int64_t off = ((int64_t(b) * p.Lkv + j0 + jj) * p.Hk + hk) * D + d;
        if constexpr (BF16) {
          kx = feature_t<POLY>(bf16_to_f32(static_cast<const uint16_t*>(p.k)[off]), p.phi_k);
          vx = bf16_to_f32(static_cast<const uint16_t*>(p.v)[off]);
        } else {
          kx = feature_t<POLY>(static_cast<const float*>(p.k)[off], p.phi_k);
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

// Delta pass on the matrix cores (bf16 models).  dS^T = V^T phi(K) over the
// split's tokens with v_mfma_f32_32x32x16_bf16: A = V^T (d_out x tokens),
// B = phi(K) (tokens x d_in).  phi is applied in float32 to the bf16 keys
// and fed as a bf16 hi + lo pair (two MFMAs), so the products keep ~16
// significant bits; V is exact in bf16.  64-token tiles of K and V are
// staged row-major in LDS with the 16-byte chunk of row r at chunk
// position c ^ swz(r); both operands are then read "transposed" (8
// consecutive tokens of one channel per lane) with ds_read_b64_tr_b16.
// Wavefront w owns d_in block w % (D/32) and (D/32)^2 / 4 blocks of d_out.
typedef short dl_i16x4 __attribute__((ext_vector_type(4)));
typedef short dl_i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) dl_i16x4 dl_lds_i16x4;
constexpr int kMDeltaBN = 64;  // tokens per LDS tile

template <int D>
__device__ __forceinline__ int dswz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Three workgroups per CU (<= 168 registers): more tile loads in flight for
// this memory-bound pass.  POLY: the caller's cubic feature map (a template
// parameter, so the map costs no branch per element).
template <int D, bool POLY>
__global__ __launch_bounds__(256, 3) void hybrid_delta_mfma_kernel(HybridStateLaunch p) {
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int ROWB = 2 * D;              // bytes per token row
  constexpr int NB = D / 32;               // 32-channel blocks
  constexpr int MBW = NB * NB / 4;         // d_out blocks per wavefront
  __shared__ __attribute__((aligned(16))) char kt[kMDeltaBN * ROWB];
  __shared__ __attribute__((aligned(16))) char vt[kMDeltaBN * ROWB];

  // blockIdx.x = ((c * nsplit + s) * B + b) * Hk + hk
  int64_t bid = blockIdx.x;
  const int hk = int(bid % p.Hk); bid /= p.Hk;
  const int b = int(bid % p.B); bid /= p.B;
  const int s = int(bid % p.nsplit);
  const int64_t c = bid / p.nsplit;
  int64_t c0, c1;
  hybrid_delta_range(p, c, &c0, &c1);
  const int64_t per = (c1 - c0 + p.nsplit - 1) / p.nsplit;
  const int64_t t0 = min(c1, c0 + s * per), t1 = min(c1, t0 + per);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int nb = wave % NB;                // d_in block
  const int mb0 = (wave / NB) * MBW;       // first d_out block

  // transposed-read address of block db (see the attention kernel's V^T reads)
  auto tr_addr = [&](int db) {
    const int s16 = lane & 15, rho = s16 >> 2, q4 = s16 & 3;
    const int rowo = 8 * g + rho;
    const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * q4;
    return uint32_t(rowo * ROWB + (((d >> 3) ^ dswz<D>(rowo)) * 16) + (d & 7) * 2);
  };
  const uint32_t kaddr = tr_addr(nb);
  uint32_t vaddr[MBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i) vaddr[i] = tr_addr(mb0 + i);
  auto tr8 = [&](const char* base, uint32_t addr, int kk) {
    const dl_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dl_lds_i16x4*)(base + addr + (16 * kk) * ROWB));
    const dl_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dl_lds_i16x4*)(base + addr + (16 * kk + 4) * ROWB));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 acc[MBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  float zacc = 0.f;
  const int64_t tok_stride = int64_t(p.Hk) * D;  // elements between tokens
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t(b) * p.Lkv * p.Hk + hk) * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t(b) * p.Lkv * p.Hk + hk) * D;

  // tile loads run one tile ahead in registers: tile j+1 is in flight while
  // tile j is on the matrix cores.  Rows past the split's end load row 0 of
  // the tile (which exists) and are zeroed when the tile is written to LDS
  // (not at the load, which would wait for the data right there); their
  // key rows also get phi = 0 in the product below.
  constexpr int NCH = kMDeltaBN * CPR / 256;  // 16-byte chunks per thread per tile
  static_assert(NCH * 256 == kMDeltaBN * CPR, "tile chunks per thread");
  uint4 kpre[NCH], vpre[NCH];
  // chunk c of a thread: row tid / CPR + c * (256 / CPR) of the tile, 16-byte
  // chunk tid % CPR of the row
  const int row0 = tid / CPR;
  const int64_t lane_off = int64_t(row0) * tok_stride + (tid % CPR) * 8;
  auto gload = [&](int64_t j0) {
    const int nv = int(min<int64_t>(kMDeltaBN, t1 - j0));
    const uint16_t* kb = kg + j0 * tok_stride;
    const uint16_t* vb = vg + j0 * tok_stride;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int64_t off = row0 + c * (256 / CPR) < nv ? lane_off + c * (256 / CPR) * tok_stride : (tid % CPR) * 8;
      kpre[c] = *reinterpret_cast<const uint4*>(kb + off);
      vpre[c] = *reinterpret_cast<const uint4*>(vb + off);
    }
  };
  if (t0 < t1) gload(t0);
  for (int64_t j0 = t0; j0 < t1; j0 += kMDeltaBN) {
    const int nv = int(min<int64_t>(kMDeltaBN, t1 - j0));
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = tid + 256 * c, row = e / CPR, ch = e % CPR;
      const int at = row * ROWB + ((ch ^ dswz<D>(row)) * 16);
      const uint32_t m = row < nv ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(kt + at) = make_uint4(kpre[c].x & m, kpre[c].y & m, kpre[c].z & m, kpre[c].w & m);
      *reinterpret_cast<uint4*>(vt + at) = make_uint4(vpre[c].x & m, vpre[c].y & m, vpre[c].z & m, vpre[c].w & m);
    }
    __syncthreads();
    if (j0 + kMDeltaBN < t1) gload(j0 + kMDeltaBN);
#pragma unroll
    for (int kk = 0; kk < kMDeltaBN / 16; ++kk) {
      if (16 * kk >= nv) break;
      // B = phi(K) for tokens 16kk + 8g + j, channel 32nb + lane%32
      const dl_i16x8 kr = tr8(kt, kaddr, kk);
      bf16x8 bh, bl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float f = feature_t<POLY>(bf16_to_f32(static_cast<uint16_t>(kr[j])), p.phi_k);
        if (16 * kk + 8 * g + j >= nv) f = 0.f;
        zacc += f;
        const __bf16 h = static_cast<__bf16>(f);
        bh[j] = h;
        bl[j] = static_cast<__bf16>(f - static_cast<float>(h));
      }
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, tr8(vt, vaddr[i], kk));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc[i], 0, 0, 0);
      }
    }
  }
  const int64_t slot = ((c * p.nsplit + s) * p.B + b) * p.Hk + hk;
  float* ds = p.ds + slot * D * D;
  const int r = lane & 31;
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 8 * (e / 4) + 4 * g + (e % 4);  // accumulator row of register e
      ds[int64_t(32 * (mb0 + i) + m) * D + 32 * nb + r] = acc[i][e];
    }
  // dz: each lane summed 8 of every 16 tokens of channel 32nb + r
  zacc += __shfl_xor(zacc, 32);
  if (wave < NB && g == 0) p.dz[slot * D + 32 * nb + r] = zacc;
}

// Scan pass: each lane walks the chunks for four adjacent elements of one
// (batch, kv head) state -- [D][D] dS^T elements, then the D of z -- with
// 16-byte delta loads, eight (chunk, split) slots in flight at a time.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void hybrid_scan_kernel(HybridStateLaunch p) {
  constexpr int NE = D * D + D;  // elements per (batch, kv head): S^T, then z
  constexpr int NV = NE / 4;
  static_assert((D * D) % 4 == 0 && D % 4 == 0, "float4 groups stay in S or z");
  const int64_t gt = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t bh = gt / NV;
  if (bh >= int64_t(p.B) * p.Hk) return;
  const int e = int(gt % NV) * 4;
  const bool is_z = e >= D * D;
  const int zi = e - D * D;            // first z element (is_z)
  const int dout = e / D, din = e % D;  // first S^T element (!is_z): din .. din + 3
  float run[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.zero_in) {
    // a new sequence: the incoming state is zero and is not read
  } else if (is_z) {
    const float4 z4 = *reinterpret_cast<const float4*>(p.z_in + bh * D + zi);
    run[0] = z4.x; run[1] = z4.y; run[2] = z4.z; run[3] = z4.w;
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) run[u] = p.s_in[bh * D * D + int64_t(din + u) * D + dout];  // s is [d_in][d_out]
  }
  const float* dsrc = is_z ? p.dz + bh * D + zi : p.ds + bh * D * D + e;
  const int64_t dstep = int64_t(p.B) * p.Hk * (is_z ? D : D * D);  // between (chunk, split) slots
  auto store = [&](int64_t c) {
    const int64_t cs = c * p.B * p.Hk + bh;  // [c][b][hk]
    if (is_z) {
      *reinterpret_cast<float4*>(p.zc + cs * D + zi) = make_float4(run[0], run[1], run[2], run[3]);
    } else if constexpr (BF16) {
      uint2 w;
      w.x = pack_bf16x2(run[0], run[1]);
      w.y = pack_bf16x2(run[2], run[3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.sc) + cs * D * D + e) = w;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.sc) + cs * D * D + e) = make_float4(run[0], run[1], run[2], run[3]);
    }
  };
  // The (chunk, split) slots in order, eight loads in flight: a chunk's
  // delta is the sum of its splits (in split order), and its prefix is
  // stored before the delta is added.
  const int64_t nsl = p.n_chunks * p.nsplit;
  float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = 0;
  int64_t c = 0;
  for (int64_t j0 = 0; j0 < nsl; j0 += 8) {
    float4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = min(j0 + u, nsl - 1);  // past the end: the last slot again (in bounds, unused)
      x[u] = *reinterpret_cast<const float4*>(dsrc + j * dstep);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < nsl) {
        d.x += x[u].x; d.y += x[u].y; d.z += x[u].z; d.w += x[u].w;
        if (++s == p.nsplit) {
          store(c);
          run[0] += d.x; run[1] += d.y; run[2] += d.z; run[3] += d.w;
          d = make_float4(0.f, 0.f, 0.f, 0.f);
          s = 0;
          ++c;
        }
      }
    }
  }
  if (is_z) {
    *reinterpret_cast<float4*>(p.z_out + bh * D + zi) = make_float4(run[0], run[1], run[2], run[3]);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) p.s_out[bh * D * D + int64_t(din + u) * D + dout] = run[u];
  }
}

template <int D, bool BF16>
hipError_t launch_d(const HybridStateLaunch& p, hipStream_t s) {
  const int64_t nblk = p.n_chunks * p.nsplit * p.B * p.Hk;
  if (nblk > 0) {
    const dim3 grid(static_cast<unsigned>(nblk));
    if constexpr (BF16) {
      if (p.phi_k.poly) hipLaunchKernelGGL((hybrid_delta_mfma_kernel<D, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((hybrid_delta_mfma_kernel<D, false>), grid, dim3(256), 0, s, p);
    } else {
      if (p.phi_k.poly) hipLaunchKernelGGL((hybrid_delta_kernel<D, BF16, true>), grid, dim3(kDeltaThreads), 0, s, p);
      else hipLaunchKernelGGL((hybrid_delta_kernel<D, BF16, false>), grid, dim3(kDeltaThreads), 0, s, p);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t nthr = int64_t(p.B) * p.Hk * ((D * D + D) / 4);
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
