// attn_mfma.hip -- bf16 flash attention on the gfx950 matrix cores.
//
// Exact softmax attention O = softmax(scale Q K^T) V per head, the
// "standard FlashAttention" step the pages run per frame / per ring step
// (FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
// Transformers, Sec. 3.3; ReGenVC: End-to-End Real-Time Generative Video
// Coding at Ultra-Low Bitrate, USP paragraph), with three epilogues: plain,
// ring (log-sum-exp fold into a float32 running partial) and chunk-hybrid
// (joint normalisation with the linear-attention partial of MobileWan:
// Closing the Quality Gap for Mobile Video Diffusion, review of Sec. 3.2).
//
// gfx950 design
//  * Transposed scores.  Each wavefront owns QB blocks of 32 queries and
//    computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the queries sit on
//    the MFMA N axis (one query per lane column), keys on M.  A lane then
//    holds 16 keys of one query per 32x32 block, so the softmax row max is a
//    reduction inside the lane plus one exchange with lane^32, and the row
//    rescale factor of the output is a per-lane scalar.
//  * Key permutation.  The K rows fed to the MFMA A operand are permuted
//    (bits 2 and 3 of the row index swapped) so that the S^T accumulator
//    registers 8h..8h+7 of a lane hold 8 consecutive keys.  Converted to
//    bf16 they are directly the B operand of O^T = V^T P^T -- no shuffles
//    between the two matrix products.
//  * Q stays in registers for the whole kernel; K and V tiles of 64 keys
//    are double-buffered in LDS (K row-major, V transposed to V^T[d][key]
//    while it is written), both XOR-swizzled so the 16-byte operand reads
//    of a wavefront are bank-conflict free.  The next tile's global loads
//    are issued before the current tile's math and land in LDS after it:
//    one barrier per tile.
//  * Online softmax in log2 units (scale*log2(e) folded into one FMA before
//    v_exp_f32); the running sum stays per lane and is combined with lane^32
//    once at the end.
//  * Workgroup ids are remapped so each of the 8 XCDs walks a contiguous
//    range of (head, query-tile) work and its L2 serves one head's K/V.
#include "attn_epilogue.hpp"
#include "vdit_internal.hpp"

namespace vdit {
namespace {

constexpr int kBN = 64;  // keys per LDS tile

__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// 16-bit element e (0..7) of a 16-byte vector
__device__ __forceinline__ uint32_t elem16(const uint4& u, int e) {
  const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D, int QB, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attn_mfma_kernel(AttnLaunch p, int64_t total) {
  constexpr int NT = 64 * NW;
  constexpr int WQ = 32 * QB;       // queries per wavefront
  constexpr int BM = NW * WQ;       // queries per workgroup
  constexpr int NCH = D / 8;        // 16-byte chunks per K row
  constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int KPT = kBN * NCH / NT;  // keys per thread when loading a tile
  constexpr int TILE = kBN * D;     // bf16 elements of one K (or V^T) tile
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "tile load mapping");
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r = lane & 31;

  // ---------------------------------------------------------------- work --
  const int64_t lid = xcd_remap(blockIdx.x, total);
  const bool hybrid = p.epi == kEpiHybrid;
  int64_t q_begin, q_end, chunk_id = 0;
  int h, b, nseg;
  KvSeg hseg;  // the chunk's own keys (hybrid)
  if (!hybrid) {
    const int64_t tiles = (p.Lq + BM - 1) / BM;
    const int64_t qt = lid % tiles, rest = lid / tiles;
    h = int(rest % p.Hq);
    b = int(rest / p.Hq);
    q_begin = qt * BM;
    q_end = min(p.Lq, q_begin + BM);
    nseg = p.nseg;
  } else {
    const int64_t tpc = (p.chunk + BM - 1) / BM;
    const int64_t t = lid % tpc, rest = lid / tpc;
    chunk_id = rest % p.n_chunks;
    const int64_t rest2 = rest / p.n_chunks;
    h = int(rest2 % p.Hq);
    b = int(rest2 / p.Hq);
    const int64_t c0 = chunk_id * p.chunk;
    const int64_t c1 = min(p.Lq, c0 + p.chunk);
    q_begin = c0 + t * BM;
    q_end = min(c1, q_begin + BM);
    if (q_begin >= q_end) return;
    nseg = 1;
    hseg.k = static_cast<const uint16_t*>(p.hk) + c0 * p.Hk * D;
    hseg.v = static_cast<const uint16_t*>(p.hv) + c0 * p.Hk * D;
    hseg.len = c1 - c0;
    hseg.bstride = p.Lq * p.Hk * D;
  }
  // segment descriptors are read from the kernel argument block (uniform)
  auto seg_at = [&](int si) -> KvSeg { return hybrid ? hseg : p.seg[si]; };
  const int hk = h / (p.Hq / p.Hk);

  // ------------------------------------------------------------ Q in VGPRs --
  bf16x8 Qr[QB][KS];
  const int64_t qw0 = q_begin + wave * WQ;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t qrow = qw0 + 32 * qb + r;
    const bool ok = qrow < q_end;
    const uint16_t* src = static_cast<const uint16_t*>(p.q) + ((int64_t(b) * p.Lq + (ok ? qrow : q_begin)) * p.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = *reinterpret_cast<const uint4*>(src + 16 * ks + 8 * g);
      if (!ok) u = make_uint4(0, 0, 0, 0);
      Qr[qb][ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 O[DB][QB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[db][qb][i] = 0.f;
  float m2[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m2[qb] = -INFINITY; lsum[qb] = 0.f; }

  // ------------------------------------------------------ tile bookkeeping --
  int ntiles = 0;
  for (int s = 0; s < nseg; ++s) ntiles += int((seg_at(s).len + kBN - 1) / kBN);

  const int lrow0 = KPT * (tid / NCH);  // first key row this thread loads
  const int lch = tid % NCH;            // 16-byte chunk (8 channels) it loads
  uint4 kreg[KPT], vreg[KPT];

  auto load_tile = [&](int si, int64_t j0) {
    const KvSeg sg = seg_at(si);
    const int64_t nv = sg.len - j0;
    const uint16_t* kb = static_cast<const uint16_t*>(sg.k) + int64_t(b) * sg.bstride + int64_t(hk) * D + lch * 8;
    const uint16_t* vb = static_cast<const uint16_t*>(sg.v) + int64_t(b) * sg.bstride + int64_t(hk) * D + lch * 8;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = lrow0 + u;
      if (key < nv) {
        const int64_t off = (j0 + key) * p.Hk * D;
        kreg[u] = *reinterpret_cast<const uint4*>(kb + off);
        vreg[u] = *reinterpret_cast<const uint4*>(vb + off);
      } else {
        kreg[u] = make_uint4(0, 0, 0, 0);
        vreg[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* Kl = lds + buf * 2 * TILE;
    uint16_t* Vl = Kl + TILE;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = lrow0 + u;
      const int phys = lch ^ (swap_bits23(key & 31) & (NCH - 1));
      *reinterpret_cast<uint4*>(Kl + key * D + phys * 8) = kreg[u];
    }
    // V^T[d][key]: KPT consecutive keys of one channel per store
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = lch * 8 + e;
      const int phys = (lrow0 >> 3) ^ ((d + (d >> 3)) & 7);
      uint16_t* dst = Vl + d * kBN + phys * 8 + (lrow0 & 7);
      if constexpr (KPT == 2) {
        *reinterpret_cast<uint32_t*>(dst) = elem16(vreg[0], e) | (elem16(vreg[1], e) << 16);
      } else if constexpr (KPT == 4) {
        uint2 w;
        w.x = elem16(vreg[0], e) | (elem16(vreg[1], e) << 16);
        w.y = elem16(vreg[2], e) | (elem16(vreg[3], e) << 16);
        *reinterpret_cast<uint2*>(dst) = w;
      } else {
        uint4 w;
        w.x = elem16(vreg[0], e) | (elem16(vreg[1], e) << 16);
        w.y = elem16(vreg[2], e) | (elem16(vreg[3], e) << 16);
        w.z = elem16(vreg[4], e) | (elem16(vreg[5], e) << 16);
        w.w = elem16(vreg[6], e) | (elem16(vreg[7], e) << 16);
        *reinterpret_cast<uint4*>(dst) = w;
      }
    }
  };

  const float c2 = p.scale_log2;
  int cur_s = 0;
  int64_t cur_j = 0;
  int64_t cur_len = 0;
  if (ntiles > 0) {
    while (seg_at(cur_s).len == 0) ++cur_s;
    cur_len = seg_at(cur_s).len;
    load_tile(cur_s, cur_j);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int nv = int(min<int64_t>(kBN, cur_len - cur_j));
    // next tile
    int nxt_s = cur_s;
    int64_t nxt_j = cur_j + kBN;
    int64_t nxt_len = cur_len;
    if (t + 1 < ntiles) {
      if (nxt_j >= nxt_len) {
        nxt_j = 0;
        ++nxt_s;
        while (seg_at(nxt_s).len == 0) ++nxt_s;
        nxt_len = seg_at(nxt_s).len;
      }
      load_tile(nxt_s, nxt_j);
    }

    const uint16_t* Kl = lds + (t & 1) * 2 * TILE;
    const uint16_t* Vl = Kl + TILE;

    // S^T = K Q^T for two 32-key blocks
    f32x16 S[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][qb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = 32 * kb + swap_bits23(r);
        const int phys = (2 * ks + g) ^ (swap_bits23(row & 31) & (NCH - 1));
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kl + row * D + phys * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Qr[qb][ks], S[kb][qb], 0, 0, 0);
      }
    }
    if (nv < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kb + 16 * (i >> 3) + 8 * g + (i & 7);
          if (key >= nv) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) S[kb][qb][i] = -INFINITY;
          }
        }
    }

    // online softmax (log2 units), P^T in bf16 as the next B operands
    bf16x8 P[2][QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[kb][qb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m2[qb], mx * c2);
      const float alpha = fast_exp2(m2[qb] - mn);
      m2[qb] = mn;
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[db][qb][i] *= alpha;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 pv;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float e = fast_exp2(fmaf(S[kb][qb][8 * hh + j], c2, -mn));
            ls += e;
            pv[j] = static_cast<__bf16>(e);
          }
          P[kb][qb][hh] = pv;
        }
      lsum[qb] += ls;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + r;
        const int phys = (2 * kk + g) ^ ((d + (d >> 3)) & 7);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vl + d * kBN + phys * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[kk >> 1][qb][kk & 1], O[db][qb], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
    cur_s = nxt_s;
    cur_j = nxt_j;
    cur_len = nxt_len;
  }

  // -------------------------------------------------------------- epilogue --
  float inv[QB], lse_s[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lsum[qb] + __shfl_xor(lsum[qb], 32);
    inv[qb] = lt > 0.f ? 1.f / lt : 0.f;
    lse_s[qb] = partial_lse(m2[qb], lt);
  }

  if (p.epi == kEpiPlain || p.epi == kEpiRing) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int64_t q = qw0 + 32 * qb + r;
      if (q >= q_end) continue;
      const int64_t orow = ((int64_t(b) * p.Lq + q) * p.Hq + h) * D;
      const int64_t lrow = (int64_t(b) * p.Hq + h) * p.Lq + q;
      float wa = 0.f, wb = inv[qb], lse_out = lse_s[qb];
      const bool merge_prev = p.epi == kEpiRing && p.has_prev;
      if (merge_prev) {
        const MergeW w = merge_weights(p.part_lse[lrow], lse_s[qb]);
        wa = w.wa;
        wb = w.wb * inv[qb];
        lse_out = w.lse;
      }
      const bool to_part = p.epi == kEpiRing && !p.final_out;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = 32 * db + 8 * i4 + 4 * g;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = O[db][qb][4 * i4 + e] * wb;
          if (merge_prev) {
            const float4 pv = *reinterpret_cast<const float4*>(p.part_o + orow + d);
            y[0] = fmaf(wa, pv.x, y[0]); y[1] = fmaf(wa, pv.y, y[1]);
            y[2] = fmaf(wa, pv.z, y[2]); y[3] = fmaf(wa, pv.w, y[3]);
          }
          if (to_part) {
            *reinterpret_cast<float4*>(p.part_o + orow + d) = make_float4(y[0], y[1], y[2], y[3]);
          } else {
            uint2 w;
            w.x = pack_bf16x2(y[0], y[1]);
            w.y = pack_bf16x2(y[2], y[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + orow + d) = w;
          }
        }
      if (g == 0) {
        if (to_part) p.part_lse[lrow] = lse_out;
        else if (p.lse) p.lse[lrow] = lse_out;
      }
    }
    return;
  }

  // chunk-hybrid: O_lin^T = S_c^T phi(Q)^T on the matrix cores (S_c^T held as
  // bf16 hi + lo planes), den = phi(q)^T z_c in float32
  const int64_t sidx = (chunk_id * p.B + b) * p.Hk + hk;
  const int64_t plane = p.n_chunks * p.B * p.Hk * D * D;
  const uint16_t* st_hi = static_cast<const uint16_t*>(p.st) + sidx * D * D;
  const uint16_t* st_lo = st_hi + plane;
  const float* z = p.zc + sidx * D;
  float den[QB];
  bf16x8 Fq[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float dn = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 za = *reinterpret_cast<const float4*>(z + 16 * ks + 8 * g);
      const float4 zb = *reinterpret_cast<const float4*>(z + 16 * ks + 8 * g + 4);
      const float zz[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
      bf16x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = phi_elu1(static_cast<float>(Qr[qb][ks][j]));
        dn = fmaf(x, zz[j], dn);
        f[j] = static_cast<__bf16>(x);
      }
      Fq[qb][ks] = f;
    }
    den[qb] = dn + __shfl_xor(dn, 32);
  }
  MergeW w[QB];
  float inv_den[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lse_l = den[qb] > 0.f ? logf(den[qb]) : -INFINITY;
    w[qb] = merge_weights(lse_s[qb], lse_l);
    inv_den[qb] = den[qb] > 0.f ? 1.f / den[qb] : 0.f;
  }
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 A[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) A[qb][i] = 0.f;
    const int dout = 32 * db + r;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(st_hi + dout * D + 16 * ks + 8 * g);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(st_lo + dout * D + 16 * ks + 8 * g);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        A[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, Fq[qb][ks], A[qb], 0, 0, 0);
        A[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, Fq[qb][ks], A[qb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int64_t q = qw0 + 32 * qb + r;
      if (q >= q_end) continue;
      const int64_t orow = ((int64_t(b) * p.Lq + q) * p.Hq + h) * D;
      const float ws = w[qb].wa * inv[qb], wl = w[qb].wb * inv_den[qb];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * g;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = ws * O[db][qb][4 * i4 + e] + wl * A[qb][4 * i4 + e];
        uint2 u;
        u.x = pack_bf16x2(y[0], y[1]);
        u.y = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + orow + d) = u;
      }
    }
  }
  if (p.lse && g == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int64_t q = qw0 + 32 * qb + r;
      if (q < q_end) p.lse[(int64_t(b) * p.Hq + h) * p.Lq + q] = w[qb].lse;
    }
  }
}

template <int D, int QB, int NW>
hipError_t launch_cfg(const AttnLaunch& p, hipStream_t s) {
  constexpr int BM = NW * 32 * QB;
  int64_t total;
  if (p.epi == kEpiHybrid) total = ((p.chunk + BM - 1) / BM) * p.n_chunks * p.Hq * p.B;
  else total = ((p.Lq + BM - 1) / BM) * p.Hq * p.B;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_mfma_kernel<D, QB, NW>), dim3(static_cast<unsigned>(total)), dim3(64 * NW), 0, s, p, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnLaunch& p, hipStream_t s) {
  // Large query sets: 64 queries per wavefront (each K/V operand read from
  // LDS feeds two MFMAs).  Small ones (one frame of a stream, short chunks):
  // 32 per wavefront so the grid still covers the 256 CUs.
  const int64_t rows = (p.epi == kEpiHybrid ? p.chunk : p.Lq);
  const int64_t work256 = ((rows + 255) / 256) * p.Hq * p.B * (p.epi == kEpiHybrid ? p.n_chunks : 1);
  const bool big = work256 >= 512;
  if (p.D == 128) return big ? launch_cfg<128, 2, 4>(p, s) : launch_cfg<128, 1, 4>(p, s);
  return big ? launch_cfg<64, 2, 4>(p, s) : launch_cfg<64, 1, 4>(p, s);
}

}  // namespace vdit
