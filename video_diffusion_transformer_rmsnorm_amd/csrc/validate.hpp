// validate.hpp -- argument validation for the vdit C ABI.
//
// Header-only and free of HIP calls so that a plain host compiler can build
// it for CPU-only tests.  Every check runs before any launch; on failure the
// caller writes nothing and reports the returned message.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <string>

namespace vdit {

enum class Check { ok = 0, invalid = 1, unsupported = 2 };

struct CheckResult {
  Check code = Check::ok;
  std::string msg;
  static CheckResult good() { return {}; }
  static CheckResult bad(const std::string& m) { return {Check::invalid, m}; }
  static CheckResult unsup(const std::string& m) { return {Check::unsupported, m}; }
  explicit operator bool() const { return code == Check::ok; }
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

inline size_t esize(int dtype) { return dtype == 1 ? 4 : 2; }

inline CheckResult check_dtype(int dtype) {
  if (dtype != 0 && dtype != 1) return CheckResult::bad("dtype must be VDIT_BF16 (0) or VDIT_F32 (1)");
  return CheckResult::good();
}

inline CheckResult check_head_dim(int32_t D) {
  if (D <= 0 || (D & 1)) return CheckResult::bad("head_dim must be a positive even number");
  if (D != 64 && D != 128) return CheckResult::unsup("head_dim must be 64 or 128");
  return CheckResult::good();
}

inline CheckResult check_heads(int32_t Hq, int32_t Hk) {
  if (Hq <= 0 || Hk <= 0) return CheckResult::bad("n_heads and n_kv_heads must be positive");
  if (Hq % Hk != 0) return CheckResult::bad("n_heads must be a multiple of n_kv_heads");
  return CheckResult::good();
}

struct GridArgs {
  int32_t T, H, W, pairs_t, pairs_h, pairs_w;
  float theta;
};

// v_in / v_out: the values that vdit_rope_qkv passes through (NULL for
// vdit_rope_qk).
inline CheckResult check_rope(const void* q_in, const void* k_in, const void* q_out,
                              const void* k_out, int32_t B, int64_t L, int32_t Hq, int32_t Hk,
                              int32_t D, int dtype, const GridArgs* g, int64_t token0,
                              float eps, const void* v_in = nullptr, const void* v_out = nullptr) {
  if (auto r = check_dtype(dtype); !r) return r;
  if (auto r = check_head_dim(D); !r) return r;
  if (!g) return CheckResult::bad("grid is NULL");
  if (B < 0 || L < 0) return CheckResult::bad("B and L must be non-negative");
  if ((q_in == nullptr) != (q_out == nullptr))
    return CheckResult::bad("q_in and q_out must both be set or both be NULL");
  if ((k_in == nullptr) != (k_out == nullptr))
    return CheckResult::bad("k_in and k_out must both be set or both be NULL");
  if ((v_in == nullptr) != (v_out == nullptr))
    return CheckResult::bad("v_in and v_out must both be set or both be NULL");
  if (q_in && Hq <= 0) return CheckResult::bad("n_heads must be positive when q is given");
  if (k_in && Hk <= 0) return CheckResult::bad("n_kv_heads must be positive when k is given");
  if (v_in && Hk <= 0) return CheckResult::bad("n_kv_heads must be positive when v is given");
  if (g->T <= 0 || g->H <= 0 || g->W <= 0) return CheckResult::bad("grid T, H, W must be positive");
  if (g->pairs_t < 0 || g->pairs_h < 0 || g->pairs_w < 0)
    return CheckResult::bad("rotary pair counts must be non-negative");
  if (int64_t(g->pairs_t) + g->pairs_h + g->pairs_w != D / 2)
    return CheckResult::bad("pairs_t + pairs_h + pairs_w must equal head_dim / 2");
  if (!(g->theta > 1.0f)) return CheckResult::bad("theta must be > 1");
  if (!(eps >= 0.0f)) return CheckResult::bad("eps must be >= 0");
  if (token0 < 0) return CheckResult::bad("token0 must be >= 0");
  // one workgroup holds a token's q, k (and v) rows: at most 2048 16-byte
  // pieces ((n_heads + n_kv_heads [+ n_kv_heads]) * head_dim / 8), i.e. 128
  // heads of dim 128
  if ((int64_t(q_in ? Hq : 0) + (k_in ? Hk : 0) + (v_in ? Hk : 0)) * (D / 8) > 2048)
    return CheckResult::unsup(
        "too many heads per token for the rotary kernel (n_heads + n_kv_heads, plus n_kv_heads with values, "
        "<= 16384 / head_dim)");
  const int64_t cells = int64_t(g->T) * g->H * g->W;
  if (token0 + L > cells) return CheckResult::bad("token0 + L exceeds the T*H*W grid");
  for (const void* p : {q_in, k_in, q_out, k_out, v_in, v_out})
    if (p && !aligned16(p)) return CheckResult::bad("tensor pointers must be 16-byte aligned");
  const size_t es = esize(dtype);
  const size_t nq = q_in ? size_t(B) * size_t(L) * size_t(Hq) * size_t(D) * es : 0;
  const size_t nk = k_in ? size_t(B) * size_t(L) * size_t(Hk) * size_t(D) * es : 0;
  const size_t nv = v_in ? size_t(B) * size_t(L) * size_t(Hk) * size_t(D) * es : 0;
  if (q_in && q_out != q_in && overlaps(q_in, nq, q_out, nq))
    return CheckResult::bad("q_out partially overlaps q_in");
  if (k_in && k_out != k_in && overlaps(k_in, nk, k_out, nk))
    return CheckResult::bad("k_out partially overlaps k_in");
  if (q_out && k_out && overlaps(q_out, nq, k_out, nk))
    return CheckResult::bad("q_out overlaps k_out");
  if (v_in) {
    // the values' output may only be the values' input itself (in place):
    // any other overlap with a tensor of the call is rejected
    if (v_out != v_in && overlaps(v_in, nv, v_out, nv)) return CheckResult::bad("v_out partially overlaps v_in");
    if ((q_in && overlaps(v_out, nv, q_in, nq)) || (q_out && overlaps(v_out, nv, q_out, nq)) ||
        (k_in && overlaps(v_out, nv, k_in, nk)) || (k_out && overlaps(v_out, nv, k_out, nk)))
      return CheckResult::bad("v_out overlaps q or k");
    if ((q_out && overlaps(q_out, nq, v_in, nv)) || (k_out && overlaps(k_out, nk, v_in, nv)))
      return CheckResult::bad("q_out or k_out overlaps v_in");
  }
  return CheckResult::good();
}

inline CheckResult check_rms_norm(const void* x_in, const void* x_out, int32_t B, int64_t L,
                                  int32_t H, int32_t D, int dtype, const float* gain, float eps) {
  if (auto r = check_dtype(dtype); !r) return r;
  if (auto r = check_head_dim(D); !r) return r;
  if (B < 0 || L < 0) return CheckResult::bad("B and L must be non-negative");
  if (H <= 0) return CheckResult::bad("n_heads must be positive");
  const bool empty = int64_t(B) * L == 0;  // nothing to read or write: NULL allowed
  if (!empty && (!x_in || !x_out)) return CheckResult::bad("x_in and x_out must be set");
  if (!(eps >= 0.0f)) return CheckResult::bad("eps must be >= 0");
  if (!aligned16(x_in) || !aligned16(x_out) || (gain && !aligned16(gain)))
    return CheckResult::bad("tensor and gain pointers must be 16-byte aligned");
  const size_t n = size_t(B) * size_t(L) * size_t(H) * size_t(D) * esize(dtype);
  if (x_out != x_in && overlaps(x_in, n, x_out, n)) return CheckResult::bad("x_out partially overlaps x_in");
  return CheckResult::good();
}

// Mirror of vdit_attn_args with plain types (kept layout-identical).
struct AttnArgs {
  int32_t mode, dtype, B, n_heads, n_kv_heads, head_dim;
  int64_t Lq, Lkv;
  float scale;
  int32_t n_kv_chunks;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* const* k_chunks;
  const void* const* v_chunks;
  const int64_t* chunk_len;
  void* k_cache;
  void* v_cache;
  int64_t frame;
  int32_t n_slots;
  uint32_t flags;
  int64_t chunk_tokens;
  float* state_s;
  float* state_z;
  void* workspace;
  size_t workspace_bytes;
  int64_t overlap_tokens;
  int64_t ctx_tokens;
  float key_norm_max;
  int32_t reserved1;
  const float* phi_coef;
};

constexpr uint32_t kAttnRingFold = 1u;   // VDIT_ATTN_RING_FOLD
constexpr uint32_t kAttnStateZero = 2u;  // VDIT_ATTN_STATE_ZERO

constexpr int kMaxRingChunks = 64;

// Workspace layout of the chunk-hybrid mode (byte offsets from the workspace
// base, each region 256-byte aligned):
//   dS   [n_chunks][nsplit][B][Hk][D][D] float32   per-split chunk state deltas (transposed: [d_out][d_in])
//   dz   [n_chunks][nsplit][B][Hk][D]    float32
//   S_c  [n_chunks][B][Hk][D][D]         float32 (F32 path) or bf16 (BF16 path, half the area), transposed
//   z_c  [n_chunks][B][Hk][D]            float32
struct HybridLayout {
  int64_t n_chunks = 0;
  int nsplit = 1;
  size_t off_ds = 0, off_dz = 0, off_sc = 0, off_zc = 0, total = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int hybrid_nsplit(int64_t chunk_tokens, int64_t n_chunks, int64_t B, int64_t Hk) {
  // token splits per chunk: enough (chunk, split, batch, head) workgroups for
  // about 512 in total (two per CU), each split >= 64 tokens, at most 8
  const int64_t units = n_chunks * B * Hk;
  int64_t s = units > 0 ? (512 + units - 1) / units : 1;
  if (s > chunk_tokens / 64) s = chunk_tokens / 64;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return int(s);
}

inline HybridLayout hybrid_layout(const AttnArgs& a) {
  HybridLayout h;
  const int64_t L = a.Lq, C = a.chunk_tokens;
  const size_t D = size_t(a.head_dim), B = size_t(a.B), Hk = size_t(a.n_kv_heads);
  h.n_chunks = C > 0 ? (L + C - 1) / C : 0;
  h.nsplit = hybrid_nsplit(C, h.n_chunks, a.B, a.n_kv_heads);
  const size_t nc = size_t(h.n_chunks), ns = size_t(h.nsplit);
  size_t off = 0;
  h.off_ds = off; off = align256(off + nc * ns * B * Hk * D * D * 4);
  h.off_dz = off; off = align256(off + nc * ns * B * Hk * D * 4);
  h.off_sc = off; off = align256(off + nc * B * Hk * D * D * 4);  // f32 (bf16 uses half)
  h.off_zc = off; off = align256(off + nc * B * Hk * D * 4);
  h.total = off;
  return h;
}

inline size_t ring_workspace_bytes(const AttnArgs& a) {
  if (a.n_kv_chunks <= 1) return 0;
  const size_t o = size_t(a.B) * size_t(a.Lq) * size_t(a.n_heads) * size_t(a.head_dim) * 4;
  const size_t l = size_t(a.B) * size_t(a.n_heads) * size_t(a.Lq) * 4;
  return align256(o) + align256(l);
}

// Key split of FULL / ROLLING bf16 attention.  When the 128-query
// workgroups of a call would not give each of the device's `cus` compute
// units two of them -- or when a call of several rounds of them would end
// on a round at most half full (more than three per CU in all, so a call
// that the three-per-CU shape fits in one round keeps it; at least 8192
// keys), in which case the keys are cut in two and the rounds double with
// a fuller last one -- the keys are cut into nsplit ranges of split_keys keys
// (a multiple of the 64-key tile, each range at least 256 keys, at most 8
// ranges); every range yields a float32 partial (normalised O and its LSE)
// and a merge pass combines them.
struct SplitPlan {
  int nsplit = 1;
  int64_t split_keys = 0;
};

inline SplitPlan split_plan(int dtype, int64_t B, int64_t Lq, int64_t Hq, int64_t keys, int cus) {
  SplitPlan s;
  if (dtype != 0 || B <= 0 || Lq <= 0 || Hq <= 0 || keys <= 0 || cus <= 0) return s;
  const int64_t wg = ((Lq + 127) / 128) * Hq * B;
  const int64_t target = 2 * int64_t(cus);
  int64_t n;
  if (wg >= target) {
    const int64_t rem = wg % target;  // workgroups of the last round
    if (wg <= 3 * int64_t(cus) || rem == 0 || 2 * rem > target || keys < 8192) return s;
    n = 2;
  } else {
    n = (target + wg - 1) / wg;
  }
  if (n > 8) n = 8;
  if (n > keys / 256) n = keys / 256;
  if (n < 2) return s;
  const int64_t per = ((keys + n - 1) / n + 63) / 64 * 64;
  n = (keys + per - 1) / per;
  if (n < 2) return s;
  s.nsplit = int(n);
  s.split_keys = per;
  return s;
}

inline size_t split_workspace_bytes(const SplitPlan& s, int64_t B, int64_t Lq, int64_t Hq, int64_t D) {
  if (s.nsplit < 2) return 0;
  const size_t n = size_t(s.nsplit);
  return align256(n * size_t(B) * size_t(Lq) * size_t(Hq) * size_t(D) * 4) +
         align256(n * size_t(B) * size_t(Hq) * size_t(Lq) * 4);
}

// Keys one FULL / ROLLING call attends to.
inline int64_t attn_keys(const AttnArgs& a) {
  if (a.mode == 2) {
    const int64_t nvalid = a.frame + 1 < a.n_slots ? a.frame + 1 : a.n_slots;
    return nvalid * a.Lq;
  }
  return a.Lkv;
}

// flags and the hybrid's polynomial feature maps
inline CheckResult check_attn_options(const AttnArgs& a) {
  if (a.flags & ~(kAttnRingFold | kAttnStateZero)) return CheckResult::bad("unknown attention flags");
  if ((a.flags & kAttnRingFold) && a.mode != 1) return CheckResult::bad("VDIT_ATTN_RING_FOLD belongs to RING");
  if ((a.flags & kAttnStateZero) && a.mode != 3)
    return CheckResult::bad("VDIT_ATTN_STATE_ZERO belongs to CHUNK_HYBRID");
  if (a.phi_coef) {
    if (a.mode != 3) return CheckResult::bad("phi_coef belongs to CHUNK_HYBRID (NULL otherwise)");
    for (int i = 0; i < 8; ++i)
      if (!std::isfinite(a.phi_coef[i])) return CheckResult::bad("phi_coef must be finite");
  }
  return CheckResult::good();
}

// A device range one call touches: written ranges (outputs, caches, the
// state, the workspace) may overlap no other range of the call; ranges that
// are only read may overlap each other.
struct Region {
  const void* p;
  size_t n;
  const char* name;
  bool written;
};

inline CheckResult check_disjoint(const Region* r, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < i; ++j)
      if ((r[i].written || r[j].written) && overlaps(r[i].p, r[i].n, r[j].p, r[j].n))
        return CheckResult::bad(std::string(r[i].name) + " overlaps " + r[j].name);
  return CheckResult::good();
}

// Aliasing and workspace placement of an attention call (run after the
// mode's own checks, before anything is launched): the workspace, when given,
// is 16-byte aligned and, like o, lse, the rolling caches and the hybrid
// state, overlaps none of the call's other tensors.  The one permitted
// alias: a ROLLING call with B = 1 may pass the cache slot itself as k / v
// (the insert is then skipped).
inline CheckResult check_attn_regions(const AttnArgs& a) {
  const size_t es = esize(a.dtype), D = size_t(a.head_dim), B = size_t(a.B);
  const size_t nq = B * size_t(a.Lq) * size_t(a.n_heads) * D * es;
  const size_t nl = B * size_t(a.n_heads) * size_t(a.Lq) * 4;
  const size_t row = size_t(a.n_kv_heads) * D * es;  // bytes per key of one batch
  if (a.workspace && a.workspace_bytes > 0 && !aligned16(a.workspace))
    return CheckResult::bad("workspace must be 16-byte aligned");
  Region r[2 * kMaxRingChunks + 8];
  int n = 0;
  r[n++] = {a.q, nq, "q", false};
  r[n++] = {a.o, nq, "o", true};
  if (a.lse) r[n++] = {a.lse, nl, "lse", true};
  if (a.workspace) r[n++] = {a.workspace, a.workspace_bytes, "workspace", true};
  switch (a.mode) {
    case 0:
    case 3: {
      const size_t nk = B * size_t(a.Lkv) * row;
      r[n++] = {a.k, nk, "k", false};
      r[n++] = {a.v, nk, "v", false};
      if (a.mode == 3) {
        r[n++] = {a.state_s, B * size_t(a.n_kv_heads) * D * D * 4, "state_s", true};
        r[n++] = {a.state_z, B * size_t(a.n_kv_heads) * D * 4, "state_z", true};
      }
      break;
    }
    case 1:
      for (int c = 0; c < a.n_kv_chunks && c < kMaxRingChunks; ++c) {
        r[n++] = {a.k_chunks[c], B * size_t(a.chunk_len[c]) * row, "a key chunk", false};
        r[n++] = {a.v_chunks[c], B * size_t(a.chunk_len[c]) * row, "a value chunk", false};
      }
      break;
    case 2: {
      const size_t frame = size_t(a.Lq) * row;  // one slot of one batch
      const size_t nc = size_t(a.n_slots) * B * frame;
      r[n++] = {a.k_cache, nc, "k_cache", true};
      r[n++] = {a.v_cache, nc, "v_cache", true};
      const int64_t slot = a.n_slots > 0 ? a.frame % a.n_slots : 0;
      for (int which = 0; which < 2; ++which) {
        const void* src = which ? a.v : a.k;
        const char* cache = static_cast<const char*>(which ? a.v_cache : a.k_cache);
        if (!src) continue;
        if (cache && src == cache + size_t(slot) * frame) {
          if (a.B == 1) continue;  // the slot itself: nothing to copy
          return CheckResult::bad("ROLLING: k / v may be the cache slot only when B = 1");
        }
        r[n++] = {src, B * frame, which ? "v" : "k", false};
      }
      break;
    }
  }
  return check_disjoint(r, n);
}

inline CheckResult check_attn(const AttnArgs& a) {
  if (auto r = check_dtype(a.dtype); !r) return r;
  if (auto r = check_head_dim(a.head_dim); !r) return r;
  if (auto r = check_heads(a.n_heads, a.n_kv_heads); !r) return r;
  if (a.B < 0 || a.Lq < 0 || a.Lkv < 0) return CheckResult::bad("B, Lq, Lkv must be non-negative");
  if (a.mode < 0 || a.mode > 3) return CheckResult::bad("unknown attention mode");
  if (!(a.scale == a.scale)) return CheckResult::bad("scale is NaN");
  const size_t es = esize(a.dtype);
  const size_t D = size_t(a.head_dim);
  const size_t nq = size_t(a.B) * size_t(a.Lq) * size_t(a.n_heads) * D * es;
  const bool empty_q = (a.B == 0 || a.Lq == 0);
  if (!empty_q) {
    if (!a.q || !a.o) return CheckResult::bad("q and o must be non-NULL");
    if (!aligned16(a.q) || !aligned16(a.o)) return CheckResult::bad("q and o must be 16-byte aligned");
  }
  if (a.lse && !aligned16(a.lse)) return CheckResult::bad("lse must be 16-byte aligned");
  if (!empty_q && overlaps(a.q, nq, a.o, nq)) return CheckResult::bad("o overlaps q");
  if (!(a.key_norm_max >= 0.f) || !std::isfinite(a.key_norm_max))
    return CheckResult::bad("key_norm_max must be finite and >= 0");
  if (a.mode != 3 && (a.overlap_tokens != 0 || a.ctx_tokens != 0))
    return CheckResult::bad("overlap_tokens and ctx_tokens belong to CHUNK_HYBRID (0 otherwise)");
  if (auto r = check_attn_options(a); !r) return r;
  switch (a.mode) {
    case 0: {  // FULL
      if (a.Lkv > 0 && !empty_q) {
        if (!a.k || !a.v) return CheckResult::bad("k and v must be non-NULL");
        if (!aligned16(a.k) || !aligned16(a.v)) return CheckResult::bad("k and v must be 16-byte aligned");
        const size_t nk = size_t(a.B) * size_t(a.Lkv) * size_t(a.n_kv_heads) * D * es;
        if (overlaps(a.o, nq, a.k, nk) || overlaps(a.o, nq, a.v, nk))
          return CheckResult::bad("o overlaps k or v");
      }
      break;
    }
    case 1: {  // RING
      if (a.n_kv_chunks < 1) return CheckResult::bad("RING needs n_kv_chunks >= 1");
      if (a.n_kv_chunks > kMaxRingChunks) return CheckResult::unsup("too many ring chunks (max 64)");
      if (!a.k_chunks || !a.v_chunks || !a.chunk_len)
        return CheckResult::bad("RING needs k_chunks, v_chunks and chunk_len");
      int64_t sum = 0;
      for (int c = 0; c < a.n_kv_chunks; ++c) {
        if (a.chunk_len[c] < 0) return CheckResult::bad("chunk_len must be non-negative");
        sum += a.chunk_len[c];
        if (a.chunk_len[c] > 0 && !empty_q) {
          if (!a.k_chunks[c] || !a.v_chunks[c]) return CheckResult::bad("RING chunk pointer is NULL");
          if (!aligned16(a.k_chunks[c]) || !aligned16(a.v_chunks[c]))
            return CheckResult::bad("RING chunk pointers must be 16-byte aligned");
        }
      }
      if (sum != a.Lkv) return CheckResult::bad("chunk_len must sum to Lkv");
      const size_t need = ring_workspace_bytes(a);
      if (need && !empty_q) {
        if (!a.workspace || a.workspace_bytes < need)
          return CheckResult::bad("RING workspace too small (see vdit_attn_workspace_bytes)");
      }
      break;
    }
    case 2: {  // ROLLING
      if (a.n_slots < 1) return CheckResult::bad("ROLLING needs n_slots >= 1");
      if (a.frame < 0) return CheckResult::bad("frame must be >= 0");
      if (!empty_q) {
        if (!a.k_cache || !a.v_cache) return CheckResult::bad("ROLLING needs k_cache and v_cache");
        if (!aligned16(a.k_cache) || !aligned16(a.v_cache))
          return CheckResult::bad("caches must be 16-byte aligned");
        if ((a.k == nullptr) != (a.v == nullptr))
          return CheckResult::bad("ROLLING: k and v must both be set or both be NULL");
        if (!aligned16(a.k) || !aligned16(a.v)) return CheckResult::bad("k and v must be 16-byte aligned");
        const size_t nc = size_t(a.n_slots) * size_t(a.B) * size_t(a.Lq) * size_t(a.n_kv_heads) * D * es;
        if (overlaps(a.o, nq, a.k_cache, nc) || overlaps(a.o, nq, a.v_cache, nc))
          return CheckResult::bad("o overlaps a cache");
        if (overlaps(a.k_cache, nc, a.v_cache, nc)) return CheckResult::bad("k_cache overlaps v_cache");
      }
      break;
    }
    case 3: {  // CHUNK_HYBRID
      if (a.chunk_tokens < 1) return CheckResult::bad("CHUNK_HYBRID needs chunk_tokens >= 1");
      if (a.overlap_tokens < 0) return CheckResult::bad("overlap_tokens must be >= 0");
      if (a.ctx_tokens < 0 || a.ctx_tokens > a.overlap_tokens)
        return CheckResult::bad("ctx_tokens must lie in [0, overlap_tokens]");
      if (a.Lkv != a.ctx_tokens + a.Lq)
        return CheckResult::bad("CHUNK_HYBRID: Lkv must equal ctx_tokens + Lq");
      if (!a.state_s || !a.state_z) return CheckResult::bad("CHUNK_HYBRID needs state_s and state_z");
      if (!aligned16(a.state_s) || !aligned16(a.state_z))
        return CheckResult::bad("state buffers must be 16-byte aligned");
      if (!empty_q) {
        if (!a.k || !a.v) return CheckResult::bad("k and v must be non-NULL");
        if (!aligned16(a.k) || !aligned16(a.v)) return CheckResult::bad("k and v must be 16-byte aligned");
        const size_t need = hybrid_layout(a).total;
        if (!a.workspace || a.workspace_bytes < need)
          return CheckResult::bad("CHUNK_HYBRID workspace too small (see vdit_attn_workspace_bytes)");
      }
      break;
    }
  }
  return check_attn_regions(a);
}

// Key-norm bound of the bounded-score softmax (bf16): 64 partial maxima per
// (batch, kv head), and per chunk in the chunk-hybrid and ring modes.
// Optional in every mode.
constexpr int kKeyBoundParts = 64;
inline size_t kbound_bytes(const AttnArgs& a) {
  if (a.dtype != 0) return 0;
  const size_t runs = a.mode == 3   ? size_t(hybrid_layout(a).n_chunks)
                      : a.mode == 1 ? size_t(a.n_kv_chunks > 1 ? a.n_kv_chunks : 1)
                                    : 1;
  return align256(runs * size_t(a.B) * size_t(a.n_kv_heads) * kKeyBoundParts * 4);
}

// Bytes of a workspace that mode requires (RING with several chunks,
// CHUNK_HYBRID); FULL and ROLLING require none.
inline size_t attn_required_bytes(const AttnArgs& a) {
  switch (a.mode) {
    case 1: return ring_workspace_bytes(a);
    case 3: return hybrid_layout(a).total;
    default: return 0;
  }
}

// Workspace of one call on a device with `cus` compute units: the required
// part, then the key-norm bound, then (FULL, ROLLING) the key-split
// partials.  Everything past the required part is optional and used when
// the workspace holds it.
// RING (bf16, 2..kRingOneLaunchMax chunks) in one launch: every chunk's float32
// partial at once (work items chunk x query tile x head, so the last round
// of workgroups is less empty than with one launch per chunk), then the
// split merge.  Optional: without room for the partials the chunks are
// folded one launch at a time into the required running partial.
constexpr int kRingOneLaunchMax = 8;  // key segments one attention launch takes
inline bool ring_one_launch(const AttnArgs& a) {
  return a.mode == 1 && a.dtype == 0 && a.n_kv_chunks >= 2 && a.n_kv_chunks <= kRingOneLaunchMax &&
         !(a.flags & kAttnRingFold);
}
inline size_t ring_partials_bytes(const AttnArgs& a) {
  if (!ring_one_launch(a)) return 0;
  SplitPlan s;
  s.nsplit = a.n_kv_chunks;
  return split_workspace_bytes(s, a.B, a.Lq, a.n_heads, a.head_dim);
}

inline size_t attn_workspace_bytes(const AttnArgs& a, int cus) {
  size_t n = attn_required_bytes(a) + kbound_bytes(a);
  if (a.mode == 0 || a.mode == 2)
    n += split_workspace_bytes(split_plan(a.dtype, a.B, a.Lq, a.n_heads, attn_keys(a), cus), a.B, a.Lq,
                               a.n_heads, a.head_dim);
  n += ring_partials_bytes(a);
  return n;
}

// Workspace check that ignores the workspace fields themselves (used by
// vdit_attn_workspace_bytes, which is called before a workspace exists).
inline CheckResult check_attn_shape(const AttnArgs& a) {
  AttnArgs b = a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  b.q = b.k = b.v = nullptr;
  b.o = nullptr;
  b.lse = nullptr;
  b.k_cache = b.v_cache = nullptr;
  b.Lq = a.Lq;
  if (auto r = check_dtype(b.dtype); !r) return r;
  if (auto r = check_head_dim(b.head_dim); !r) return r;
  if (auto r = check_heads(b.n_heads, b.n_kv_heads); !r) return r;
  if (b.B < 0 || b.Lq < 0 || b.Lkv < 0) return CheckResult::bad("B, Lq, Lkv must be non-negative");
  if (b.mode < 0 || b.mode > 3) return CheckResult::bad("unknown attention mode");
  if (b.mode == 1 && (b.n_kv_chunks < 1 || b.n_kv_chunks > kMaxRingChunks))
    return CheckResult::bad("RING needs 1 <= n_kv_chunks <= 64");
  if (b.mode == 3 && b.chunk_tokens < 1) return CheckResult::bad("CHUNK_HYBRID needs chunk_tokens >= 1");
  return check_attn_options(b);
}

inline CheckResult check_merge(const void* o_a, const float* lse_a, const void* o_b,
                               const float* lse_b, const void* o_out, const float* lse_out,
                               int in_dtype, int out_dtype, int32_t B, int64_t L, int32_t H,
                               int32_t D) {
  if (auto r = check_dtype(in_dtype); !r) return r;
  if (auto r = check_dtype(out_dtype); !r) return r;
  if (auto r = check_head_dim(D); !r) return r;
  if (B < 0 || L < 0 || H <= 0) return CheckResult::bad("B, L must be >= 0 and n_heads > 0");
  if (B == 0 || L == 0) return CheckResult::good();
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out) return CheckResult::bad("merge pointers must be non-NULL");
  for (const void* p : {o_a, static_cast<const void*>(lse_a), o_b, static_cast<const void*>(lse_b), o_out})
    if (!aligned16(p)) return CheckResult::bad("merge pointers must be 16-byte aligned");
  if (lse_out && !aligned16(lse_out)) return CheckResult::bad("lse_out must be 16-byte aligned");
  const size_t nin = size_t(B) * size_t(L) * size_t(H) * size_t(D) * esize(in_dtype);
  const size_t nout = size_t(B) * size_t(L) * size_t(H) * size_t(D) * esize(out_dtype);
  const size_t nl = size_t(B) * size_t(L) * size_t(H) * 4;
  for (const void* in : {o_a, o_b}) {
    if (in == o_out) {
      if (in_dtype != out_dtype) return CheckResult::bad("in-place merge needs in_dtype == out_dtype");
    } else if (overlaps(in, nin, o_out, nout)) {
      return CheckResult::bad("o_out partially overlaps an input");
    }
  }
  if (lse_out) {
    for (const float* in : {lse_a, lse_b})
      if (in != lse_out && overlaps(in, nl, lse_out, nl))
        return CheckResult::bad("lse_out partially overlaps an input");
    if (overlaps(lse_out, nl, o_out, nout)) return CheckResult::bad("lse_out overlaps o_out");
  }
  return CheckResult::good();
}

}  // namespace vdit
