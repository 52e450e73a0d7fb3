// vdit_internal.hpp -- kernel parameter blocks and launcher entry points
// shared between the C ABI (abi.cpp) and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace vdit {

constexpr int kMaxSeg = 8;

// A run of keys/values: element (b, j, hk, d) of a segment lives at
// base + b * bstride + (j * Hk + hk) * D + d.
struct KvSeg {
  const void* k;
  const void* v;
  int64_t len;
  int64_t bstride;  // elements between batches
};

// Feature map of the chunk-hybrid's linear term: elu(x) + 1, or (poly set)
// the cubic c[0] + c[1] x + c[2] x^2 + c[3] x^3, element-wise.
struct FeatureMap {
  float c[4];
  int32_t poly;
};

enum Epilogue : int32_t {
  kEpiPlain = 0,   // write normalised O (+ LSE)
  kEpiRing = 1,    // fold into / out of a float32 running partial
  kEpiHybrid = 2,  // merge with the linear-attention partial of the chunk
};

struct AttnLaunch {
  const void* q;
  void* o;
  float* lse;
  int64_t Lq;
  int32_t B, Hq, Hk, D;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int32_t nseg;
  int32_t epi;
  KvSeg seg[kMaxSeg];
  // ring epilogue
  float* part_o;     // [B, Lq, Hq, D] float32 running partial
  float* part_lse;   // [B, Hq, Lq]
  int32_t has_prev;  // part_* hold the partial of the earlier chunks
  int32_t final_out; // write o / lse (else write part_*)
  // chunk-hybrid (self-attention over q's own sequence, chunks of `chunk`
  // queries; chunk [c0, c1) attends with softmax to keys
  // [max(0, hyb_ctx + c0 - hyb_overlap), hyb_ctx + c1) of hyb_lkv keys)
  int64_t chunk;
  int64_t n_chunks;
  int64_t hyb_ctx;
  int64_t hyb_overlap;
  int64_t hyb_lkv;
  const void* st;    // per chunk state S_c^T [n_chunks][B][Hk][D][D]: bf16 or float32
  const float* zc;   // [n_chunks][B][Hk][D]
  const void* hk;    // key / value base of the whole sequence (hybrid)
  const void* hv;
  FeatureMap phi_q;  // applied to the queries (hybrid)
  // key split (plain attention): nsplit ranges of split_keys keys; range s
  // writes its partial to part_o / part_lse offset by s whole partials
  int32_t nsplit;
  int64_t split_keys;
  int32_t seg_split;  // 1: split s attends to the whole segment seg[s] (nsplit <= nseg)
  // bounded-score softmax: kbound[((r * B + b) * Hk + hk) * kbound_n + i]
  // are partial maxima of the squared norms of the keys a workgroup attends
  // to (r: its hybrid chunk, or its segment under seg_split, else 0); NULL:
  // online maximum
  const float* kbound;
  int32_t kbound_n;
  // caller's bound on max_j |k_j|^2 (key_norm_max^2), used instead of
  // kbound when kbound is null and this is > 0
  float kbound_sq;
};

// Partial maxima of squared key norms (bf16 keys), per run of part_len keys
// (part_len <= 0: one run, the whole segment), batch and kv head:
// out[((r * B + b) * Hk + hk) * kKeyBoundBlocks + i].
constexpr int kKeyBoundBlocks = 64;
hipError_t launch_key_bound(const KvSeg& seg, int32_t B, int32_t Hk, int32_t D, int64_t part_len, float* out,
                            hipStream_t s);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_attn_bf16(const AttnLaunch& p, hipStream_t s);
hipError_t launch_attn_f32(const AttnLaunch& p, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cus();

// Sets the calling thread's vdit_last_error() message; returns status.
int report_error(int status, const char* msg);

// Whether the bf16 kernel chosen for p uses the key-norm bound (p.kbound or
// p.kbound_sq); caller_bound: the caller supplies it (no pre-pass needed).
bool attn_uses_key_bound(const AttnLaunch& p, bool caller_bound);

// Merge of nsplit float32 attention partials ([nsplit][B][L][H][D] normalised
// O, [nsplit][B][H][L] LSE) into o (out_dtype) and lse (may be NULL).
struct SplitMergeLaunch {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;
  int64_t L;
  int32_t B, H, D, nsplit, out_dtype;
};
hipError_t launch_split_merge(const SplitMergeLaunch& p, hipStream_t s);

struct RopeLaunch {
  const void* q_in;
  const void* k_in;
  void* q_out;
  void* k_out;
  const float* q_gain;
  const float* k_gain;
  const void* v_in = nullptr;    // values: copied, or RMS-normalised (norm_v), not rotated
  void* v_out = nullptr;
  const float* v_gain = nullptr;
  int32_t norm_v = 0;
  int64_t L;
  int64_t token0;
  int64_t t_offset;
  int32_t B, Hq, Hk, D;
  int32_t T, H, W;
  int32_t pairs_t, pairs_h, pairs_w;
  float theta;
  float eps;
  int32_t norm_q;  // RMSNorm the q rows before rotating them
  int32_t norm_k;  // RMSNorm the k rows before rotating them
  int32_t dtype;
  double omega_base[3];  // theta^(-1 / P_axis) per axis t, h, w (filled by launch_rope)
};
hipError_t launch_rope(const RopeLaunch& p, hipStream_t s);

// Per-head RMSNorm without rotation: rows of D channels, rows = B * L * H.
struct RmsNormLaunch {
  const void* x_in;
  void* x_out;
  const float* gain;
  int64_t rows;
  int32_t D;
  float eps;
  int32_t dtype;
};
hipError_t launch_rms_norm(const RmsNormLaunch& p, hipStream_t s);

struct MergeLaunch {
  const void* o_a;
  const float* lse_a;
  const void* o_b;
  const float* lse_b;
  void* o_out;
  float* lse_out;
  int64_t L;
  int32_t B, H, D;
  int32_t in_dtype, out_dtype;
};
hipError_t launch_merge(const MergeLaunch& p, hipStream_t s);

struct HybridStateLaunch {
  const void* k;       // [B, L, Hk, D]
  const void* v;
  const float* s_in;   // [B, Hk, D, D]  (d_in, d_out)
  const float* z_in;   // [B, Hk, D]
  float* s_out;        // may equal s_in
  float* z_out;
  int32_t zero_in;     // 1: the incoming state is zero (s_in, z_in not read)
  float* ds;           // [n_chunks][nsplit][B][Hk][D][D] transposed (d_out, d_in)
  float* dz;           // [n_chunks][nsplit][B][Hk][D]
  void* sc;            // per-chunk state, transposed, bf16 or float32
  float* zc;
  int64_t L, chunk, n_chunks;  // L: query tokens (chunks are defined on them)
  int64_t Lkv, ctx, overlap;   // key tokens (= ctx + L), context keys, softmax overlap
  int32_t nsplit;
  int32_t B, Hk, D;
  int32_t dtype;       // of k, v; also selects the S_c format
  FeatureMap phi_k;    // applied to the keys
};
hipError_t launch_hybrid_state(const HybridStateLaunch& p, hipStream_t s);

// Keys whose phi(k) v^T the delta of chunk c adds to the running state: from
// the start of chunk c's softmax window to the start of the next one (the
// last chunk: to all keys but the last `overlap`, the next call's context).
// The state before chunk c then covers every key before its window.
__host__ __device__ inline void hybrid_delta_range(const HybridStateLaunch& p, int64_t c, int64_t* t0,
                                                   int64_t* t1) {
  const int64_t a = p.ctx + c * p.chunk - p.overlap;
  const int64_t e = c + 1 < p.n_chunks ? p.ctx + (c + 1) * p.chunk - p.overlap : p.Lkv - p.overlap;
  *t0 = a > 0 ? a : 0;
  *t1 = e > 0 ? e : 0;
}

}  // namespace vdit
