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
//  * Transposed scores.  Each wavefront owns 32 queries and computes
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the queries sit on the MFMA
//    N axis (one query per lane column), keys on M.  A lane holds 16 keys of
//    one query per 32x32 block, so the softmax row max is a reduction inside
//    the lane plus one exchange with lane^32, and the output rescale factor
//    is a per-lane scalar.
//  * Key permutation.  The K rows fed to the MFMA A operand are permuted
//    (bits 2 and 3 of the row index swapped) so that accumulator registers
//    8h..8h+7 of a lane hold 8 consecutive keys: converted to bf16 they are
//    directly the B operand of O^T = V^T P^T.
//  * K/V tiles of 64 keys move HBM -> LDS with buffer_load_dwordx4 ... lds
//    (no staging registers, no LDS store instructions).  Each 16-byte chunk
//    of a row is placed at an XOR-swizzled position chosen by the source
//    address, so the operand reads are bank-conflict free.  V stays
//    row-major in LDS; the transposed V^T operand is read with
//    ds_read_b64_tr_b16 (two reads per 16-key step).
//  * Software pipeline over tiles with separate K and V double buffers: in
//    iteration j the wavefront runs the softmax of tile j while the matrix
//    cores compute S^T of tile j+1, then O^T += V_j^T P_j^T; K_{j+2} and
//    V_{j+1} stream into the free buffers meanwhile.  One barrier per tile.
//    Two wavefronts share each SIMD (<= 256 VGPRs), so one's exp/max work
//    overlaps the other's matrix products; within a wavefront, exponentials
//    are packed one MFMA step after they are issued and the first V^T reads
//    of a tile are issued before its PV products start, so neither the
//    transcendental nor the LDS latency stalls the wavefront.
//  * Bounded-score softmax where a key-norm pre-pass bounds every score of
//    the wavefront's queries: p = 2^(c2 s) needs no running maximum, and
//    with Q pre-scaled by c2 the exponent comes straight from the MFMA
//    accumulator (one VALU op less per score).  Otherwise an online softmax
//    in log2 units with a lazy rescale: the running max only moves when a
//    row's tile max exceeds it by more than 8 (so p <= 2^8), which skips the
//    output rescale on almost every tile.
//  * Row sums at D = 64 (half the MFMA work per score, so the softmax VALU
//    work weighs twice as much): each packed P register is also the B
//    operand of a 16x16x32 MFMA against a constant 0/1 selector that sums
//    exactly the lane's own query, so the row sums cost four small matrix
//    products per tile instead of 32 VALU adds.  At D = 128 the matrix
//    cores are the busier pipe and the adds stay.
//  * All LDS addresses are precomputed per lane; tile and buffer offsets are
//    instruction immediates (the loop is unrolled by two over the buffer
//    parity).  Workgroup ids are remapped so each XCD walks a contiguous
//    range of (head, query-tile) work.
//  * Output rows leave through LDS: each wavefront stages its bf16 rows
//    (O^T pieces of 4 channels per lane) in its own LDS area and stores
//    whole rows, 1 KB per store instruction.  The chunk-hybrid epilogue
//    loads S_c^T and z_c into LDS by direct loads alongside the query
//    reload; it runs in its own kernel instance, in which wavefronts without
//    queries keep only their tile loads and barriers.
#include <atomic>
#include <type_traits>

#include "attn_epilogue.hpp"
#include "vdit_internal.hpp"

#ifndef VDIT_ATTN_BIG_QB
#define VDIT_ATTN_BIG_QB 1  // query blocks per wavefront for large problems (2: one wavefront per SIMD)
#endif
#ifndef VDIT_ATTN_BOUND_MIN_NW
#define VDIT_ATTN_BOUND_MIN_NW 4  // smallest workgroup shape (wavefronts) with the bounded-score path
#endif
#ifndef VDIT_ATTN_NPB
#define VDIT_ATTN_NPB 6  // exponential pairs (of 16) computed among the PV MFMAs
#endif
#ifndef VDIT_ATTN_DOT2
#define VDIT_ATTN_DOT2 0  // row sums by v_dot2_f32_bf16 over the packed bf16 p (slower: a serial accumulate)
#endif
#ifndef VDIT_ATTN_MSUM
#define VDIT_ATTN_MSUM 1  // D = 64: row sums of P on the matrix cores (16x16x32 against a 0/1 selector)
#endif
#ifndef VDIT_ATTN_VEARLY
#define VDIT_ATTN_VEARLY 4  // region A steps (from its end) over which the first V^T reads of region B are issued
#endif
#ifndef VDIT_ATTN_VEARLY64
#define VDIT_ATTN_VEARLY64 2  // the same at D = 64 (its region A has half the steps)
#endif
#ifndef VDIT_ATTN_KPREF
#define VDIT_ATTN_KPREF 3  // K operand reads issued ahead of their MFMA
#endif
#ifndef VDIT_ATTN_VPREF
#define VDIT_ATTN_VPREF 2  // V^T operand read pairs issued ahead of their MFMA
#endif
#ifndef VDIT_WIDE_ONE_ROUND
#define VDIT_WIDE_ONE_ROUND 1  // 8-wavefront workgroups for calls of one nearly full round
#endif
#ifndef VDIT_DEBUG_SYNC
#define VDIT_DEBUG_SYNC 0  // 1: self-check build, every pipeline stage ends on a full wait + barrier
#endif

namespace vdit {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBN = 64;        // keys per tile
constexpr float kLazy = 8.0f;  // rescale threshold of the running max (log2 units)
constexpr float kBoundSpan = 64.0f;  // largest 2 m_i (log2 units) of the bounded-score path

// 16 bytes per lane from a buffer resource straight into LDS at M0 + 16*lane.
// (The builtin only exists for the device pass; the host pass sees an empty
// body, as it never runs kernel code.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, lds_void* dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 0);
#endif
}

// Value of lane l ^ 32 (the other 32-lane half), via v_permlane32_swap on
// (x, x): of the two results one is this lane's own x and the other the
// partner's, so pick the one that differs (equal bits: either is correct).
__device__ __forceinline__ float other_half(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0] == u ? r[1] : r[0]);
}

__device__ __forceinline__ int swap_bits23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Chunk swizzle of K rows: a bijection of row % 16 onto the chunk XOR mask so
// that 16 lanes reading 16 different rows at one logical chunk hit 16
// distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// Chunk swizzle of V rows: the 4 rows one transposed read touches (rows
// 4i..4i+3, 64 bytes each) land in distinct quarters of the 256-byte bank space.
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// PV step at which the exponentials of the k-th of npb pairs moved among the
// PV MFMAs are issued (packed one step later), spread over the steps before
// the first one that reads the last pair (3 * db of 4 * db).
__host__ __device__ constexpr int pv_pair_step(int k, int npb, int db) { return (k * (3 * db - 1)) / npb; }
// Every moved pair is packed before its first reader: the pairs of the third
// quarter of P (the first npb - 4 moved, if any) by PV step 2 * db, the rest
// by step 3 * db.
__host__ __device__ constexpr bool pv_pairs_in_time(int npb, int db) {
  for (int k = 0; k < npb; ++k)
    if (pv_pair_step(k, npb, db) + 1 >= (k < npb - 4 ? 2 * db : 3 * db)) return false;
  return true;
}

// QB blocks of 32 queries per wavefront.  QB = 1: two wavefronts per SIMD
// (<= 256 registers each); QB = 2: one wavefront per SIMD with 512 registers,
// every K / V^T operand read from LDS feeding two MFMAs (half the LDS traffic
// per FLOP).  HYB: the chunk-hybrid instance (its own epilogue, and
// wavefronts without queries -- the tail of a chunk's last block -- skip the
// matrix work of the main loop, so their SIMD time goes to the other
// workgroup of the CU); the other modes use the plain/ring instance.  OCC:
// wavefronts per SIMD the registers are sized for (2, or 3 for the D = 64
// 4-wavefront shape on calls that fit one round at three workgroups per CU:
// at most 168 registers, a few spilled).  Second launch bound: workgroups
// per CU.
template <int D, int NW, int QB, bool HYB, int OCC = 2>
__global__ __launch_bounds__(64 * NW, OCC == 3 ? 12 / NW : (QB == 1 ? 8 : 4) / NW) void attn_mfma_kernel(AttnLaunch p,
                                                                                                         int64_t total) {
  constexpr int BM = 32 * NW * QB;  // queries per workgroup
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int KS = D / 16;        // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int ROWB = 2 * D;       // bytes per key row
  constexpr int TILE_B = kBN * ROWB;  // V tile bytes
  constexpr int RPI = 1024 / ROWB;  // V rows per direct-load instruction
  constexpr int IPW = kBN / RPI / NW;  // V direct-load instructions per wavefront per tile
  static_assert(IPW >= 1 && RPI * CPR == 64, "tile load mapping");
  // K rows are padded by one 16-byte chunk: rows land 16 bytes apart in the
  // bank space (conflict-free operand reads) and every operand address is a
  // per-lane base plus a compile-time offset.
  constexpr int KCPR = CPR + 1;                 // chunk slots per padded K row
  constexpr int KROWB = 16 * KCPR;
  constexpr int KTILE_B = kBN * KROWB;
  constexpr int KI = KTILE_B / 1024;            // K direct-load instructions per tile
  constexpr int KIW = (KI + NW - 1) / NW;       // ... per wavefront (at most)
  static_assert(KTILE_B % 1024 == 0, "padded K tile is whole 1 KB blocks");
  __shared__ __attribute__((aligned(1024))) char lds[2 * KTILE_B + 2 * TILE_B];  // K0 K1 V0 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5, r = lane & 31;

  // ---------------------------------------------------------------- work --
  // (32-bit index arithmetic: the launch keeps total below 2^31; a 64-bit
  // division is a long scalar sequence ahead of the first memory request)
  const uint32_t lid = uint32_t(xcd_remap(blockIdx.x, total));
  constexpr bool hybrid = HYB;
  int64_t q_begin, q_end, chunk_id = 0;
  int h, b;
  KvSeg sg;  // the keys/values this workgroup attends to
  float* part_o = p.part_o;
  float* part_lse = p.part_lse;
  if (!hybrid) {
    const uint32_t tiles = uint32_t((p.Lq + BM - 1) / BM);
    const uint32_t qt = lid % tiles;
    uint32_t rest = lid / tiles;
    uint32_t split = 0;
    if (p.nsplit > 1) {
      split = rest % p.nsplit;
      rest /= p.nsplit;
    }
    h = int(rest % uint32_t(p.Hq));
    b = int(rest / uint32_t(p.Hq));
    q_begin = int64_t(qt) * BM;
    q_end = min(p.Lq, q_begin + BM);
    sg = p.seg[0];
    if (p.nseg == 0) sg.len = 0;
    if (p.nsplit > 1) {
      if (p.seg_split) {  // split s attends to key segment s (a ring chunk), with its own key bound
        sg = p.seg[split];
        chunk_id = split;
      } else {  // keys [split * split_keys, +split_keys) of the segment
        const int64_t k0 = split * p.split_keys;
        const int64_t n = min(p.split_keys, sg.len - k0);
        sg.k = static_cast<const uint16_t*>(sg.k) + k0 * p.Hk * D;
        sg.v = static_cast<const uint16_t*>(sg.v) + k0 * p.Hk * D;
        sg.len = n > 0 ? n : 0;
      }
      part_o += split * (int64_t(p.B) * p.Lq * p.Hq * D);
      part_lse += split * (int64_t(p.B) * p.Hq * p.Lq);
    }
  } else {
    const uint32_t tpc = uint32_t((p.chunk + BM - 1) / BM);
    const uint32_t t = lid % tpc, rest = lid / tpc;
    chunk_id = rest % uint32_t(p.n_chunks);
    const uint32_t rest2 = rest / uint32_t(p.n_chunks);
    h = int(rest2 % uint32_t(p.Hq));
    b = int(rest2 / uint32_t(p.Hq));
    const int64_t c0 = chunk_id * p.chunk;
    const int64_t c1 = min(p.Lq, c0 + p.chunk);
    q_begin = c0 + int64_t(t) * BM;
    q_end = min(c1, q_begin + BM);
    if (q_begin >= q_end) return;
    // softmax window: the chunk's keys and the hyb_overlap keys before them
    const int64_t w0 = max<int64_t>(0, p.hyb_ctx + c0 - p.hyb_overlap), w1 = p.hyb_ctx + c1;
    sg.k = static_cast<const uint16_t*>(p.hk) + w0 * p.Hk * D;
    sg.v = static_cast<const uint16_t*>(p.hv) + w0 * p.Hk * D;
    sg.len = w1 - w0;
    sg.bstride = p.hyb_lkv * p.Hk * D;
  }
  const int hk = h / (p.Hq / p.Hk);
  const int64_t rs = int64_t(p.Hk) * ROWB;  // bytes between consecutive keys

  // ------------------------------------------------------------ Q in VGPRs --
  // (reloaded unscaled by the hybrid epilogue and by a rerun of the main loop)
  bf16x8 Qr[QB][KS];
  const int64_t qw0 = q_begin + wave * 32 * QB;
  auto load_q = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int64_t qrow = qw0 + 32 * qb + r;
      const bool ok = qrow < q_end;
      const uint16_t* src =
          static_cast<const uint16_t*>(p.q) + ((int64_t(b) * p.Lq + (ok ? qrow : q_begin)) * p.Hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 u = *reinterpret_cast<const uint4*>(src + 16 * ks + 8 * g);
        if (!ok) u = make_uint4(0, 0, 0, 0);
        Qr[qb][ks] = __builtin_bit_cast(bf16x8, u);
      }
    }
  };
  load_q();

  // ---------------------------------------------------- per-lane addresses --
  // direct loads.  K: instruction u (= wave + NW*i) fills padded slots
  // 64u + lane, i.e. row s / KCPR, chunk s % KCPR (the pad slot re-reads the
  // row's last chunk).  V: instruction u of this wavefront fills rows
  // lrow0 + u*RPI + lane/CPR, reading the chunk the swizzle puts at the slot.
  uint32_t koff[KIW], voff[IPW];
#pragma unroll
  for (int i = 0; i < KIW; ++i) {
    const int slot = 64 * (wave + NW * i) + lane;
    const int row = slot / KCPR, col = min(slot % KCPR, CPR - 1);
    koff[i] = uint32_t(row) * uint32_t(rs) + uint32_t(col * 16);
  }
  const int lrow0 = wave * IPW * RPI + lane / CPR;
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int row = lrow0 + u * RPI;
    voff[u] = uint32_t(row) * uint32_t(rs) + uint32_t(((lane % CPR) ^ swz_v<D>(row)) * 16);
  }
  // K operand of S^T: row 32kb + swap23(r), chunk 2ks + g
  const uint32_t kaddr = uint32_t(swap_bits23(r) * KROWB + g * 16);
  // V^T operand via transposed reads: in each 16-lane group, source lane
  // s = 4*rho + q reads row (16kk + 8g + 4h + rho), channels d0 + 4q .. +3
  // with d0 = 32db + 16*((lane/16)&1); the destination lane gets 4 keys of
  // channel d0 + lane%16.
  uint32_t vaddr[DB];
  {
    const int s16 = lane & 15, rho = s16 >> 2, q4 = s16 & 3;
    const int rowo = 8 * g + rho;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * q4;
      const int chunk = d >> 3;
      vaddr[db] = uint32_t(rowo * ROWB + ((chunk ^ swz_v<D>(rowo)) * 16) + (d & 7) * 2);
    }
  }

  // ---------------------------------------------------------- tile issue --
  const int len = int(sg.len);
  const int ntiles = (len + kBN - 1) / kBN;
  const char* kbase = reinterpret_cast<const char*>(sg.k) + (int64_t(b) * sg.bstride + int64_t(hk) * D) * 2;
  const char* vbase = reinterpret_cast<const char*>(sg.v) + (int64_t(b) * sg.bstride + int64_t(hk) * D) * 2;
  // Tile `tile` of K or V -> LDS buffer via buffer_load_dwordx4 ... lds.  The
  // buffer resource starts at the tile and covers only the keys that exist,
  // so rows past the end of the sequence read as zeros (their scores are
  // masked to -inf): no special tail path and no 64-bit address VGPRs.
  auto issue = [&](int tile, bool is_v, int buf) {
    const int j0 = tile * kBN;
    const char* tb = (is_v ? vbase : kbase) + int64_t(j0) * rs;
    int64_t avail = int64_t(len - 1 - j0) * rs + ROWB;  // bytes of existing keys from the tile start
    avail = avail < 0x7fffffff ? avail : 0x7fffffff;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(tb), (short)0, __builtin_amdgcn_readfirstlane(int(avail)), 0x00020000);
    if (is_v) {
      char* lb = lds + 2 * KTILE_B + buf * TILE_B + wave * IPW * 1024;
#pragma unroll
      for (int u = 0; u < IPW; ++u) buffer_load_lds16(rsrc, (lds_void*)(lb + u * 1024), voff[u]);
    } else {
      char* lb = lds + buf * KTILE_B;
#pragma unroll
      for (int i = 0; i < KIW; ++i) {
        const int u = wave + NW * i;
        if (u < KI) buffer_load_lds16(rsrc, (lds_void*)(lb + u * 1024), koff[i]);
      }
    }
  };

  // The first tiles go out before anything waits on Q (the bound below reads
  // Q's registers), so the two memory latencies overlap.
  auto issue_first = [&]() {
    issue(0, false, 0);
    issue(0, true, 0);
    if (ntiles > 1) issue(1, false, 1);
  };
  bool first_issued = false;
  if (ntiles > 0) {
    issue_first();
    first_issued = true;
  }

  // Chunk-hybrid epilogue state: S_c^T (bf16 [D][D]) and z_c of the chunk go
  // straight into LDS by direct loads, rows [0, D/2) and then z_c in K
  // buffer `kbuf`, rows [D/2, D) in V buffer 1 - kbuf, each row's 16-byte
  // chunk c at position c ^ swz_k(row) (the epilogue's operand reads of one
  // instruction then fall in distinct bank groups).
  constexpr int ST_NI = D * D * 2 / 1024;  // direct-load instructions of S_c^T
  static_assert(D * D + 1024 <= KTILE_B && D * D <= TILE_B, "S_c^T halves and z_c fit the tile buffers");
  auto issue_state = [&](int kbuf) {
    const int64_t sidx = (chunk_id * p.B + b) * p.Hk + hk;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(static_cast<const uint16_t*>(p.st) + sidx * D * D), (short)0, D * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.zc + sidx * D), (short)0, D * 4, 0x00020000);
    char* lo = lds + kbuf * KTILE_B;
    char* hi = lds + 2 * KTILE_B + (1 - kbuf) * TILE_B;
#pragma unroll
    for (int i = 0; i < (ST_NI + NW) / NW; ++i) {
      const int u = wave + NW * i;
      if (u < ST_NI) {
        const int row0 = 64 * u / CPR;  // first row of this instruction (all its rows in one half)
        const int row = row0 + lane / CPR, c = lane % CPR;
        char* dst = row0 < D / 2 ? lo + row0 * ROWB : hi + (row0 - D / 2) * ROWB;
        buffer_load_lds16(rs, (lds_void*)dst, uint32_t(row * ROWB + ((c ^ swz_k<D>(row)) * 16)));
      } else if (u == ST_NI) {
        buffer_load_lds16(rz, (lds_void*)(lo + D * D), uint32_t(lane * 16));  // lanes past z_c read zeros
      }
    }
  };

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
  // Row sums on the matrix cores (D = 64, where the VALU is the busier
  // pipe): each packed P register (16 keys of 32 queries, the B operand of
  // the PV product) is read as the B operand of a 16x16x32 MFMA, whose lane
  // l supplies keys 8 (l / 16) .. + 7 of column l % 16 -- query l % 32 of
  // the P layout, so columns mix queries n and n + 16 in alternate 8-key
  // groups.  The 0/1 selector A[m][k] = [bit 2 of m == bit 3 of k] sums, in
  // output rows 4i..4i+3, exactly the groups of query (l % 16) + 16 (i & 1),
  // which is lane l's own query: every register of the accumulator then
  // holds the lane's whole row sum (both lane halves), over every tile.
  constexpr bool MSUM = VDIT_ATTN_MSUM != 0 && D == 64;
  f32x4 lacc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 msel;
  {
    const __bf16 one = static_cast<__bf16>((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 1.0f : 0.0f);
#pragma unroll
    for (int j = 0; j < 8; ++j) msel[j] = one;
  }
  // the row's sum of p over its keys (both lane halves)
  auto row_total = [&](int qb) -> float {
    if constexpr (MSUM) return lacc[qb][0];
    else return lsum[qb] + other_half(lsum[qb]);
  };
  const float c2 = p.scale_log2;

  // Bounded scores (Cauchy-Schwarz): |s_ij| <= |q_i| |k_j| <= |q_i| Kmax,
  // with Kmax^2 the largest squared key norm from the bound pass.  m_i =
  // c2 |q_i| Kmax then bounds every score of query i in log2 units: for
  // m_i <= kBoundSpan / 2 every p = 2^(c2 s) is representable as it stands,
  // so the wavefront needs neither a running maximum nor rescaling nor a
  // shift of the scores.  A wavefront takes this path when all its queries
  // qualify; otherwise it keeps the online maximum (both paths pass the
  // same barriers).
  // (8- and 4-wavefront kernels; the 2-wavefront kernel, for problems too
  // small to fill the chip, keeps a single loop)
  bool fast = false;
  if (NW >= VDIT_ATTN_BOUND_MIN_NW && (p.kbound != nullptr || p.kbound_sq > 0.f)) {
    // the caller's bound, or the partial maxima (at most 64): one per lane,
    // then a wavefront max
    float kmax2 = p.kbound_sq;
    if (p.kbound != nullptr) {
      const float* kbp = p.kbound + ((chunk_id * p.B + b) * p.Hk + hk) * p.kbound_n;
      kmax2 = lane < p.kbound_n ? kbp[lane] : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) kmax2 = fmaxf(kmax2, __shfl_xor(kmax2, o));
    }
    bool ok = kmax2 < 3.0e38f;
    float mb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float n2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = static_cast<float>(Qr[qb][ks][j]);
          n2 = fmaf(x, x, n2);
        }
      n2 += other_half(n2);
      mb[qb] = c2 * sqrtf(n2 * kmax2);
      ok = ok && (2.f * mb[qb] <= kBoundSpan);
    }
    fast = __ballot(!ok) == 0;
    if (fast) {
      // |c2 s| <= mb <= kBoundSpan / 2 = 32: p = 2^(c2 s) lies in
      // [2^-32, 2^32] and the row's largest p is >= 2^-32, well inside the
      // float32 and bfloat16 exponent range (a row sum over fewer than 2^31
      // keys stays below 2^63).  So the scores need no shift
      // (m = 0) and, with Q pre-scaled by c2 (one more bf16 rounding of q,
      // a relative 2^-9 at most), the MFMA accumulator holds c2 s itself.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        m2[qb] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j) Qr[qb][ks][j] = static_cast<__bf16>(static_cast<float>(Qr[qb][ks][j]) * c2);
      }
    }
#if defined(__HIP_DEVICE_COMPILE__)
    // keep Q's bf16 registers where they are (reading them as floats above
    // must not change how the compiler holds them through the main loop)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(Qr[qb][ks]));
#endif
  }

  // S^T of the tile in K buffer `buf` (unmasked); each K operand feeds QB MFMAs
  auto qk = [&](int buf, f32x16 (*S)[QB]) {
    const char* Kl = lds + buf * KTILE_B + kaddr;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][qb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kl + ks * 32 + kb * 32 * KROWB);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Qr[qb][ks], S[kb][qb], 0, 0, 0);
      }
  };

  // lane-local max of one query block's 32 tile scores (a 4-level max3 tree)
  auto lane_max = [&](f32x16 (*S)[QB], int qb) -> float {
    float a[11];
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int i0 = 3 * j, i1 = 3 * j + 1, i2 = 3 * j + 2;
      a[j] = fmaxf(fmaxf(S[i0 >> 4][qb][i0 & 15], S[i1 >> 4][qb][i1 & 15]), S[i2 >> 4][qb][i2 & 15]);
    }
    a[10] = fmaxf(S[1][qb][14], S[1][qb][15]);
    const float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]), b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
    const float b2 = fmaxf(fmaxf(a[6], a[7]), a[8]), b3 = fmaxf(a[9], a[10]);
    return fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
  };

  // The tail masks must stay inside their (wavefront-uniform) branch: left
  // to itself the compiler turns them into selects at the join, one per
  // score on every tile.  An empty asm on the masked registers in the branch
  // keeps them there.
  auto pin_scores = [&](f32x16 (*S)[QB]) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(S[kb][qb]));
#endif
  };

  // row max of tile scores S (lane maxima mx precomputed on unmasked scores):
  // mask the keys >= nv of a tail tile, combine the two lane halves, then the
  // lazy rescale
  auto row_max = [&](f32x16 (*S)[QB], float* mx, int nv) {
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
      pin_scores(S);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = lane_max(S, qb);
    }
    bool grow[QB];
    float mcand[QB];
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m = fmaxf(mx[qb], other_half(mx[qb]));
      mcand[qb] = m * c2;
      grow[qb] = mcand[qb] > m2[qb] + kLazy;
      any = any || grow[qb];
    }
    if (__ballot(any)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mn = grow[qb] ? mcand[qb] : m2[qb];
        const float alpha = fast_exp2(m2[qb] - mn);
        m2[qb] = mn;
        lsum[qb] *= alpha;
        if constexpr (MSUM) lacc[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[db][qb][i] *= alpha;
      }
    }
  };

  // keys >= nv of a tail tile -> -inf (bounded-score path)
  auto mask_tail = [&](f32x16 (*S)[QB], int nv) {
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
      pin_scores(S);
    }
  };

  // The two regions of a tile: the interleave is written out in source
  // order and pinned with scheduling fences after every MFMA step, so it does
  // not depend on the scheduler's pattern matching.  Region A: step st issues
  // the K operand read for step st + KPREF, the MFMA(s) of step st, and its
  // share of this tile's exponentials; each pair of exponentials is packed to
  // bf16 and added to a running total one step after it is issued, so the
  // transcendental latency passes under the next MFMA instead of stalling the
  // wavefront; its last VEARLY steps also issue the first VPREF transposed V
  // reads of region B (the V tile is complete since the previous barrier), so
  // region B starts without waiting on LDS.  Region B: step st issues the
  // transposed V reads for step st + VPREF, the PV MFMA(s) of step st and a
  // slice of the next tile's lane maximum.
  // Exponential pairs (2 scores, one packed bf16 pair of P) of this tile:
  // pairs [0, NPA) go to region A, spread evenly over its MFMA steps; the
  // last NPB pairs (second key half) to region B, each placed before the
  // first PV step that reads it, so both regions carry similar VALU work.
  constexpr int NPAIR = 16 * QB;
  constexpr int NPB = QB == 1 ? VDIT_ATTN_NPB : 0;
  constexpr int NPA = NPAIR - NPB;
  static_assert(NPB >= 0 && NPB <= 8, "pairs moved to region B");
  float run[QB];
  // p of pair pr (2 scores of one query block) into pe.  Bounded-score
  // wavefronts hold scores already in log2 units (Q pre-scaled by c2, no
  // shift): p = 2^s straight from the accumulator.
  float pe[NPAIR][2];
  auto exp_issue = [&](int pr, f32x16 (*S)[QB], auto fastc) {
    constexpr bool FAST = decltype(fastc)::value;
    const int el = 2 * pr;
    const int qb = el >> 5, kb2 = (el >> 4) & 1, i = el & 15;
    const float x0 = S[kb2][qb][i], x1 = S[kb2][qb][i + 1];
    pe[pr][0] = fast_exp2(FAST ? x0 : fmaf(x0, c2, -m2[qb]));
    pe[pr][1] = fast_exp2(FAST ? x1 : fmaf(x1, c2, -m2[qb]));
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(pe[pr][0]), "+v"(pe[pr][1]));
#endif
  };
  // pe of pair pr -> its bf16 pair in P, and into the running sum
  auto exp_finish = [&](int pr, bf16x8 (*P)[QB][2]) {
    const int el = 2 * pr;  // (qb, kb, hh, j) in that order
    const int qb = el >> 5, kb2 = (el >> 4) & 1, i = el & 15, hh = i >> 3, j = i & 7;
    const float e0 = pe[pr][0], e1 = pe[pr][1];
    const __bf16 b0 = static_cast<__bf16>(e0), b1 = static_cast<__bf16>(e1);
    P[kb2][qb][hh][j] = b0;
    P[kb2][qb][hh][j + 1] = b1;
    if constexpr (MSUM) return;  // (the row sums come from the matrix cores)
#if VDIT_ATTN_DOT2
    // the row sum of the rounded p that the PV product uses: one v_dot2 with
    // (1, 1) per packed pair
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    run[qb] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2v{b0, b1}, bf16x2v{(__bf16)1.0f, (__bf16)1.0f}, run[qb], false);
#else
    run[qb] += e0 + e1;
#endif
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(run[qb]));  // keep the sum in this step (no sinking)
#endif
  };
  constexpr int VPB = 4 * DB;
  constexpr int VP = VDIT_ATTN_VPREF < VPB ? VDIT_ATTN_VPREF : VPB;
  constexpr int VEARLY = D == 64 ? VDIT_ATTN_VEARLY64 : VDIT_ATTN_VEARLY;
  static_assert(VEARLY >= 1 && VEARLY <= 2 * KS, "early V^T reads within region A");
  auto vread_buf = [&](int vbuf, int st) {
    const char* Vl = lds + 2 * KTILE_B + vbuf * TILE_B;
    const int kk = st / DB, db = st % DB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vl + vaddr[db] + (16 * kk) * ROWB));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vl + vaddr[db] + (16 * kk + 4) * ROWB));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto region_a = [&](int buf, f32x16 (*Sn)[QB], f32x16 (*S)[QB], bf16x8 (*P)[QB][2], auto fastc, int vbuf, i16x8* vpre) {
    constexpr int NSTEP = 2 * KS;
    constexpr int KP = VDIT_ATTN_KPREF < NSTEP ? VDIT_ATTN_KPREF : NSTEP;
    const char* Kl = lds + buf * KTILE_B + kaddr;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) Sn[kb][qb][i] = 0.f;
    bf16x8 ka[NSTEP];
#pragma unroll
    for (int st = 0; st < KP; ++st)
      ka[st] = *reinterpret_cast<const bf16x8*>(Kl + (st >> 1) * 32 + (st & 1) * 32 * KROWB);
    if constexpr (!MSUM) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) run[qb] = 0.f;
    }
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + KP < NSTEP) {
        const int sn = st + KP;
        ka[sn] = *reinterpret_cast<const bf16x8*>(Kl + (sn >> 1) * 32 + (sn & 1) * 32 * KROWB);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        Sn[st & 1][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st], Qr[qb][st >> 1], Sn[st & 1][qb], 0, 0, 0);
#pragma unroll
      for (int pr = 0; pr < NPA; ++pr)
        if (st > 0 && (pr * NSTEP) / NPA == st - 1) exp_finish(pr, P);
#pragma unroll
      for (int pr = 0; pr < NPA; ++pr)
        if ((pr * NSTEP) / NPA == st) exp_issue(pr, S, fastc);
      // the first V^T operands of region B
#pragma unroll
      for (int v = 0; v < VP; ++v)
        if (st == NSTEP - VEARLY + v * VEARLY / VP) vpre[v] = vread_buf(vbuf, v);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int pr = 0; pr < NPA; ++pr)
      if ((pr * NSTEP) / NPA == NSTEP - 1) exp_finish(pr, P);
  };
  auto region_b = [&](int buf, f32x16 (*S)[QB], bf16x8 (*P)[QB][2], f32x16 (*Sn)[QB], float* mx, auto domaxc, const i16x8* vpre) {
    constexpr bool DOMAX = decltype(domaxc)::value;
    constexpr int NSTEP = 4 * DB;
    constexpr int PER = 32 / NSTEP;  // scores of one query block folded into the max per step
    constexpr int LASTB = 3 * DB;    // first PV step that reads the last pair
    // second-half pair NPA + k: exponentials issued at step bstep(k), packed
    // at bstep(k) + 1, which comes before its first reader (PV step 2 * DB
    // for the first quarter, 3 * DB after; a step issues its MFMA first)
    auto bstep = [](int k) { return pv_pair_step(k, NPB, DB); };
    static_assert(pv_pairs_in_time(NPB, DB), "an exponential pair packed after its PV reader");
    i16x8 va[NSTEP];
    auto vread = [&](int st) { return vread_buf(buf, st); };
#pragma unroll
    for (int st = 0; st < VP; ++st) va[st] = vpre[st];
    float m[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m[qb] = -INFINITY;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + VP < NSTEP) va[st + VP] = vread(st + VP);
      const int kk = st / DB, db = st % DB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[st]), P[kk >> 1][qb][kk & 1],
                                                            O[db][qb], 0, 0, 0);
      if constexpr (MSUM) {
        if (db == DB - 1) {  // after the P register's last PV product
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(msel, P[kk >> 1][qb][kk & 1], lacc[qb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int k = 0; k < NPB; ++k)
        if (st > 0 && bstep(k) == st - 1) exp_finish(NPA + k, P);
#pragma unroll
      for (int k = 0; k < NPB; ++k)
        if (bstep(k) == st) exp_issue(NPA + k, S, std::integral_constant<bool, !DOMAX>{});
      if constexpr (DOMAX) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int x = 0; x < PER; x += 2) {
            const int el = st * PER + x;
            m[qb] = fmaxf(fmaxf(m[qb], Sn[el >> 4][qb][el & 15]), Sn[el >> 4][qb][(el & 15) + 1]);
#if defined(__HIP_DEVICE_COMPILE__)
            asm volatile("" : "+v"(m[qb]));  // keep the max in this step (no sinking)
#endif
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!MSUM) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) lsum[qb] += run[qb];
    }
    if constexpr (DOMAX) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = m[qb];
    }
  };

  auto wait_and_sync = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // Self-check build (VDIT_DEBUG_SYNC=1): the tile loads of an iteration are
  // waited for before any of its LDS reads, and each region ends on a
  // workgroup barrier, so no LDS write can overlap a read of the same bytes
  // from another stage.  Same arithmetic in the same order: its results must
  // equal the pipelined build's bit for bit.
  auto debug_sync = [&]() {
    if constexpr (VDIT_DEBUG_SYNC != 0) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };

  // A hybrid wavefront with no queries keeps only its share of the tile
  // loads and the barriers of the main loop (same count and order).
  const bool idle = HYB && qw0 >= q_end;
  auto idle_loop = [&]() {
    if (!first_issued) issue_first();
    first_issued = false;
    wait_and_sync();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int P0 = t & 1;
      if (t + 2 < ntiles) issue(t + 2, false, P0);
      if (t + 1 < ntiles) issue(t + 1, true, 1 - P0);
      debug_sync();
      debug_sync();
      debug_sync();
      wait_and_sync();
    }
  };

  auto main_loop = [&](auto fastc) {
    constexpr bool FAST = decltype(fastc)::value;
    // prologue: K_0, V_0, K_1 in flight (issued at the start for the first
    // pass); S^T of tile 0
    if (!first_issued) issue_first();
    first_issued = false;
    wait_and_sync();
    f32x16 S[2][QB];
    qk(0, S);
    float mx[QB];
    if constexpr (!FAST) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mx[qb] = lane_max(S, qb);
    }
    __syncthreads();

    auto iteration = [&](int t, auto parity) {
      constexpr int P0 = decltype(parity)::value;
      // stream K_{t+2} into K buffer P0 and V_{t+1} into V buffer 1-P0
      if (t + 2 < ntiles) issue(t + 2, false, P0);
      if (t + 1 < ntiles) issue(t + 1, true, 1 - P0);
      debug_sync();
      if constexpr (FAST) mask_tail(S, min(kBN, len - t * kBN));
      else row_max(S, mx, min(kBN, len - t * kBN));
      // region A: exps of tile t || S^T of tile t+1 (computed on the last
      // tile too, on stale LDS data, and discarded)
      f32x16 Sn[2][QB];
      bf16x8 P[2][QB][2];
      __builtin_amdgcn_sched_barrier(0);
      i16x8 vpre[VP];
      region_a(1 - P0, Sn, S, P, fastc, P0, vpre);
      debug_sync();
      // region B: O^T += V^T P^T || lane max of tile t+1's scores
      region_b(P0, S, P, Sn, mx, std::integral_constant<bool, !FAST>{}, vpre);
      debug_sync();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) S[kb][qb] = Sn[kb][qb];
      wait_and_sync();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      iteration(t, std::integral_constant<int, 0>{});
      iteration(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntiles) iteration(t, std::integral_constant<int, 0>{});
  };
  if (ntiles > 0) {
    if constexpr (NW >= VDIT_ATTN_BOUND_MIN_NW) {
      if (idle) idle_loop();
      else if (fast) main_loop(std::true_type{});
      else main_loop(std::false_type{});
      // With a true bound every p of a bounded-score row lies in
      // [2^-32, 2^32] (up to rounding), so its row sum lies in [2^-64, 2^64]
      // for fewer than 2^31 keys.  A sum outside that range means a
      // key_norm_max below the keys' real norms: the row may have overflowed
      // or lost its largest terms to underflow.  Then the whole workgroup
      // runs its tiles once more (the barriers must match), every wavefront
      // on the running maximum with its queries reloaded unscaled.  A valid
      // bound never takes this branch.  (A second pass rather than a loop
      // around the first: loop-carried accumulators would spill.)
      if (p.kbound != nullptr || p.kbound_sq > 0.f) {  // workgroup-uniform
        bool bad = false;
        if (fast && qw0 < q_end) {  // (a wave past the block's end has no rows)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float lt = row_total(qb);
            bad = bad || !(lt >= 0x1p-64f && lt <= 0x1p64f);
          }
        }
        bad = __ballot(bad) != 0;
        // the main loop ended on a barrier after its last LDS read and with
        // no tile load in flight: the tile buffers are free for the flags
        int* flags = reinterpret_cast<int*>(lds);
        if (lane == 0) flags[wave] = bad ? 1 : 0;
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) any |= flags[w];
        __syncthreads();
        if (any) {
          fast = false;
          load_q();
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            m2[qb] = -INFINITY;
            lsum[qb] = 0.f;
            lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) O[db][qb][i] = 0.f;
          }
          if (idle) idle_loop();
          else main_loop(std::false_type{});
        }
      }
    } else {
      if (idle) idle_loop();
      else main_loop(std::false_type{});
    }
  }

  // -------------------------------------------------------------- epilogue --
  // bf16 output rows leave through LDS: a lane holds 4-channel pieces of one
  // query row (O^T layout), so storing them directly would touch 32 rows per
  // instruction.  Each wavefront writes its rows into its own LDS area
  // (32 * QB rows of 2 D bytes, the 16-byte chunk c of local row rl at
  // position c ^ swz_k(rl)) and stores whole rows, 1 KB per instruction.
  static_assert(NW * 32 * QB * ROWB <= 2 * KTILE_B + 2 * TILE_B, "output staging fits the tile buffers");
  char* const ob = lds + wave * (32 * QB * ROWB);
  auto stage_piece = [&](int rl, int chunk, float y0, float y1, float y2, float y3) {
    uint2 w;
    w.x = pack_bf16x2(y0, y1);
    w.y = pack_bf16x2(y2, y3);
    *reinterpret_cast<uint2*>(ob + rl * ROWB + ((chunk ^ swz_k<D>(rl)) * 16) + g * 8) = w;
  };
  auto store_rows = [&]() {
    constexpr int RPI_O = 1024 / ROWB;  // rows per store instruction
#pragma unroll
    for (int j = 0; j < 32 * QB / RPI_O; ++j) {
      const int rl = j * RPI_O + lane / CPR, c = lane % CPR;
      const int64_t q = qw0 + rl;
      const uint4 u = *reinterpret_cast<const uint4*>(ob + rl * ROWB + ((c ^ swz_k<D>(rl)) * 16));
      if (q < q_end) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.o) + ((int64_t(b) * p.Lq + q) * p.Hq + h) * D + c * 8) = u;
    }
  };

  if constexpr (!HYB) {
    // (the main loop ended on a barrier after its last LDS read: every area is free)
    const bool merge_prev = p.epi == kEpiRing && p.has_prev;
    const bool to_part = p.epi == kEpiRing && !p.final_out;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = row_total(qb);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse_s = partial_lse(m2[qb], lt);
      const int64_t q = qw0 + 32 * qb + r;
      const bool live = q < q_end;
      const int64_t qc = live ? q : q_begin;  // rows past the end compute on a valid row, store nothing
      const int64_t orow = ((int64_t(b) * p.Lq + qc) * p.Hq + h) * D;
      const int64_t lrowi = (int64_t(b) * p.Hq + h) * p.Lq + qc;
      float wa = 0.f, wb = inv, lse_out = lse_s;
      if (merge_prev) {
        const MergeW w = merge_weights(part_lse[lrowi], lse_s);
        wa = w.wa;
        wb = w.wb * inv;
        lse_out = w.lse;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = 32 * db + 8 * i4 + 4 * g;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = O[db][qb][4 * i4 + e] * wb;
          if (merge_prev) {
            const float4 pv4 = *reinterpret_cast<const float4*>(part_o + orow + d);
            y[0] = fmaf(wa, pv4.x, y[0]); y[1] = fmaf(wa, pv4.y, y[1]);
            y[2] = fmaf(wa, pv4.z, y[2]); y[3] = fmaf(wa, pv4.w, y[3]);
          }
          if (to_part) {
            if (live) *reinterpret_cast<float4*>(part_o + orow + d) = make_float4(y[0], y[1], y[2], y[3]);
          } else {
            stage_piece(32 * qb + r, 4 * db + i4, y[0], y[1], y[2], y[3]);
          }
        }
      if (g == 0 && live) {
        if (to_part) part_lse[lrowi] = lse_out;
        else if (p.lse) p.lse[lrowi] = lse_out;
      }
    }
    if (!to_part) store_rows();
    return;
  } else {

  // chunk-hybrid: O_lin^T = S_c^T phi(Q)^T on the matrix cores (S_c^T and
  // phi(q) in bf16, float32 accumulation), den = phi(q)^T z_c in float32.
  // The tile buffers are free (the main loop ended on a barrier after its
  // last LDS read): S_c^T and z_c go into K buffer 0 and V buffer 1 while Q
  // is reloaded unscaled (the bounded-score path scaled the registers), one
  // memory latency for the three.
  issue_state(0);
  load_q();
  wait_and_sync();
  const char* s_lo = lds;
  const char* s_hi = lds + 2 * KTILE_B + TILE_B;
  const float* z = reinterpret_cast<const float*>(s_lo + D * D);
  float lse_h[QB];
  if (qw0 < q_end) {  // (a wave past the end of the chunk's last block has no rows)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = row_total(qb);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse_s = partial_lse(m2[qb], lt);
      bf16x8 Fq[KS];
      float dn = 0.f;
      auto features = [&](auto polyc) {  // the map chosen once, not per element
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const float4 za = *reinterpret_cast<const float4*>(z + 16 * ks + 8 * g);
          const float4 zb = *reinterpret_cast<const float4*>(z + 16 * ks + 8 * g + 4);
          const float zz[8] = {za.x, za.y, za.z, za.w, zb.x, zb.y, zb.z, zb.w};
          bf16x8 f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = feature_t<decltype(polyc)::value>(static_cast<float>(Qr[qb][ks][j]), p.phi_q);
            dn = fmaf(x, zz[j], dn);
            f[j] = static_cast<__bf16>(x);
          }
          Fq[ks] = f;
        }
      };
      if (p.phi_q.poly) features(std::true_type{});
      else features(std::false_type{});
      const float den = dn + other_half(dn);
      const float lse_l = den > 0.f ? logf(den) : -INFINITY;
      const MergeW w = merge_weights(lse_s, lse_l);
      const float inv_den = den > 0.f ? 1.f / den : 0.f;
      const float ws = w.wa * inv, wl = w.wb * inv_den;
      lse_h[qb] = w.lse;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x16 A;
#pragma unroll
        for (int i = 0; i < 16; ++i) A[i] = 0.f;
        const int dout = 32 * db + r;
        const char* srow = 32 * db < D / 2 ? s_lo + dout * ROWB : s_hi + (dout - D / 2) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(srow + (((2 * ks + g) ^ swz_k<D>(dout)) * 16));
          A = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Fq[ks], A, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) O[db][qb][i] = ws * O[db][qb][i] + wl * A[i];
      }
    }
  }
  __syncthreads();  // every wavefront is done with S_c^T: the areas are free for the rows
  if (qw0 >= q_end) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        stage_piece(32 * qb + r, 4 * db + i4, O[db][qb][4 * i4], O[db][qb][4 * i4 + 1], O[db][qb][4 * i4 + 2],
                    O[db][qb][4 * i4 + 3]);
    const int64_t q = qw0 + 32 * qb + r;
    if (p.lse && g == 0 && q < q_end) p.lse[(int64_t(b) * p.Hq + h) * p.Lq + q] = lse_h[qb];
  }
  store_rows();
  }  // HYB
}

template <int D, int NW, int QB, int OCC = 2>
hipError_t launch_cfg(const AttnLaunch& p, hipStream_t s) {
  const bool hyb = p.epi == kEpiHybrid;
  constexpr int BM = NW * 32 * QB;
  int64_t total;
  if (p.epi == kEpiHybrid) total = ((p.chunk + BM - 1) / BM) * p.n_chunks * p.Hq * p.B;
  else total = ((p.Lq + BM - 1) / BM) * p.Hq * p.B * (p.nsplit > 1 ? p.nsplit : 1);
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;  // (the kernel's work index is 32-bit)
  if constexpr (OCC != 2) {
    static_assert(D == 64 && NW == 4 && QB == 1, "three wavefronts per SIMD: the D = 64 4-wavefront shape only");
    if (hyb) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, QB, false, OCC>), dim3(static_cast<unsigned>(total)), dim3(64 * NW), 0,
                       s, p, total);
  } else if (hyb) {
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, QB, true>), dim3(static_cast<unsigned>(total)), dim3(64 * NW), 0, s, p,
                       total);
  } else {
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, QB, false>), dim3(static_cast<unsigned>(total)), dim3(64 * NW), 0, s, p,
                       total);
  }
  return hipGetLastError();
}

}  // namespace

int device_cus() {
  // one entry per device, filled on first use; threads that race on an empty
  // entry all store the same attribute value (relaxed atomics: no torn reads)
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

// The 8-wavefront shape holds a whole CU per workgroup: it streams each K/V
// tile into LDS once for 256 queries (half the tile traffic of two 4-wavefront
// workgroups) but its last partial round of workgroups leaves whole CUs idle,
// where 4-wavefront workgroups spread out about one per CU (half the idle
// time).  The wide shape is ~3% faster per FLOP: take it when at most 6% of
// its CU-rounds would sit idle.
bool prefer_wide(int64_t wg256, int cus) {
  // one nearly full round (a key-split decode frame: 256 workgroups on 256
  // CUs) has no ragged last round for the narrow shape to fill
  if (VDIT_WIDE_ONE_ROUND && wg256 <= int64_t(cus) && wg256 * 100 >= 94 * int64_t(cus)) return true;
  if (wg256 < 2 * int64_t(cus)) return false;
  const int64_t rounds = (wg256 + cus - 1) / cus;
  const int64_t idle = rounds * cus - wg256;  // CU-rounds left empty
  return idle * 100 <= 6 * rounds * cus;
}

}  // namespace

namespace {
// Workgroup shape of a bf16 launch: 8, 4 or 2 wavefronts (one 32-query block
// each).
int attn_waves(const AttnLaunch& p) {
  const int64_t rows = (p.epi == kEpiHybrid ? p.chunk : p.Lq);
  const int64_t units = int64_t(p.Hq) * p.B * (p.epi == kEpiHybrid ? p.n_chunks : 1) * (p.nsplit > 1 ? p.nsplit : 1);
  const int64_t wg128 = ((rows + 127) / 128) * units;
  const int64_t wg256 = ((rows + 255) / 256) * units;
  if (prefer_wide(wg256, device_cus())) return 8;
  return wg128 >= 512 ? 4 : 2;
}
}  // namespace

// The key-norm pre-pass pays for itself where each query sees many keys:
// the chunk-hybrid's 128-query workgroups see one chunk (about a thousand
// keys) and run faster on the online maximum alone, unless the caller's
// bound makes the pre-pass unnecessary.
bool attn_uses_key_bound(const AttnLaunch& p, bool caller_bound) {
  const int nw = attn_waves(p);
  if (VDIT_ATTN_BIG_QB != 1 || nw < VDIT_ATTN_BOUND_MIN_NW) return false;
  return nw == 8 || p.epi != kEpiHybrid || caller_bound;
}

hipError_t launch_attn_bf16(const AttnLaunch& p, hipStream_t s) {
  // Workgroup shape by problem size: 256 queries (8 wavefronts) when its
  // rounds of workgroups come out nearly even; else 128 queries
  // (4 wavefronts, two workgroups per CU); else, for problems too small to
  // give every CU two such workgroups, 64 queries.
  const int64_t rows = (p.epi == kEpiHybrid ? p.chunk : p.Lq);
  const int64_t units = int64_t(p.Hq) * p.B * (p.epi == kEpiHybrid ? p.n_chunks : 1) * (p.nsplit > 1 ? p.nsplit : 1);
  const int64_t wg128 = ((rows + 127) / 128) * units;
  const int64_t wg256 = ((rows + 255) / 256) * units;
  const bool wide = prefer_wide(wg256, device_cus());
  if (p.D == 128) {
    if constexpr (VDIT_ATTN_BIG_QB == 2)
      if (wg256 >= 512) return launch_cfg<128, 4, 2>(p, s);
    if (wide) return launch_cfg<128, 8, 1>(p, s);
    return wg128 >= 512 ? launch_cfg<128, 4, 1>(p, s) : launch_cfg<128, 2, 1>(p, s);
  }
  if constexpr (VDIT_ATTN_BIG_QB == 2)
    if (wg256 >= 512) return launch_cfg<64, 4, 2>(p, s);
  if (wide) return launch_cfg<64, 8, 1>(p, s);
  // more than one round of 4-wavefront workgroups at two per CU, but one
  // round at three: the registers sized for three (the XL decode frame's 696
  // workgroups: 1.36 rounds -> 1, 7% faster; larger calls, with several
  // rounds either way, run faster at two)
  const int64_t cus = device_cus();
  if (p.epi != kEpiHybrid && wg128 > 2 * cus && wg128 <= 3 * cus) return launch_cfg<64, 4, 1, 3>(p, s);
  return wg128 >= 512 ? launch_cfg<64, 4, 1>(p, s) : launch_cfg<64, 2, 1>(p, s);
}

}  // namespace vdit
