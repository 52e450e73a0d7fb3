// abi.cpp -- the extern "C" boundary of libvdit: validation, mode dispatch
// and error reporting.  Declared in include/vdit.h.
#include "vdit.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>

#include "validate.hpp"
#include "vdit_internal.hpp"

static_assert(sizeof(vdit_attn_args) == sizeof(vdit::AttnArgs), "vdit_attn_args layout mirror");
static_assert(vdit::kRingOneLaunchMax <= vdit::kMaxSeg, "one ring launch: a segment per chunk");
static_assert(vdit::kKeyBoundParts == vdit::kKeyBoundBlocks && vdit::kKeyBoundBlocks <= 64,
              "key-bound partials: one per lane of a wavefront");
static_assert(offsetof(vdit_attn_args, workspace_bytes) == offsetof(vdit::AttnArgs, workspace_bytes),
              "vdit_attn_args layout mirror");
static_assert(offsetof(vdit_attn_args, ctx_tokens) == offsetof(vdit::AttnArgs, ctx_tokens),
              "vdit_attn_args layout mirror");
static_assert(offsetof(vdit_attn_args, key_norm_max) == offsetof(vdit::AttnArgs, key_norm_max),
              "vdit_attn_args layout mirror");
static_assert(offsetof(vdit_attn_args, flags) == offsetof(vdit::AttnArgs, flags), "vdit_attn_args layout mirror");
static_assert(offsetof(vdit_attn_args, phi_coef) == offsetof(vdit::AttnArgs, phi_coef),
              "vdit_attn_args layout mirror");
static_assert(VDIT_ATTN_RING_FOLD == vdit::kAttnRingFold, "flag mirror");
static_assert(VDIT_ATTN_STATE_ZERO == vdit::kAttnStateZero, "flag mirror");

namespace {

thread_local std::string g_last_error;

vdit_status fail(vdit_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

vdit_status from_check(const vdit::CheckResult& r) {
  if (r) return VDIT_OK;
  return fail(r.code == vdit::Check::unsupported ? VDIT_ERR_UNSUPPORTED : VDIT_ERR_INVALID_ARG, r.msg);
}

vdit_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return VDIT_OK;
  return fail(VDIT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

const vdit::AttnArgs& mirror(const vdit_attn_args* a) {
  return *reinterpret_cast<const vdit::AttnArgs*>(a);
}

float softmax_scale(const vdit::AttnArgs& a) {
  return a.scale > 0.f ? a.scale : 1.0f / std::sqrt(float(a.head_dim));
}

vdit::AttnLaunch base_launch(const vdit::AttnArgs& a) {
  vdit::AttnLaunch p;
  std::memset(&p, 0, sizeof(p));
  p.q = a.q;
  p.o = a.o;
  p.lse = a.lse;
  p.Lq = a.Lq;
  p.B = a.B;
  p.Hq = a.n_heads;
  p.Hk = a.n_kv_heads;
  p.D = a.head_dim;
  p.scale = softmax_scale(a);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.epi = vdit::kEpiPlain;
  return p;
}

hipError_t launch_attn(const vdit::AttnLaunch& p, int dtype, hipStream_t s) {
  return dtype == VDIT_BF16 ? vdit::launch_attn_bf16(p, s) : vdit::launch_attn_f32(p, s);
}

// phi_q (first = 0) or phi_k (first = 4) of a hybrid call: elu + 1 when the
// caller gives no coefficients.
vdit::FeatureMap feature_map(const float* coef, int first) {
  vdit::FeatureMap f;
  std::memset(&f, 0, sizeof(f));
  if (coef) {
    f.poly = 1;
    for (int i = 0; i < 4; ++i) f.c[i] = coef[first + i];
  }
  return f;
}

// Optional workspace area [off, off + bytes): usable when the caller's
// workspace holds it, else NULL.  (Its alignment and placement were checked
// with the other arguments, before anything was enqueued.)
char* optional_area(const vdit::AttnArgs& a, size_t off, size_t bytes) {
  if (bytes == 0 || !a.workspace || a.workspace_bytes < off + bytes) return nullptr;
  return static_cast<char*>(a.workspace) + off;
}

// Bounded-score softmax: the caller's key-norm bound when given, else the
// key-norm maxima of the launch's keys into the workspace area `area` (bf16
// only), or nothing when there is no area.
vdit_status add_key_bound(vdit::AttnLaunch& p, const vdit::KvSeg& keys, char* area, hipStream_t stream,
                          float key_norm_max, int64_t part_len = 0) {
  if (keys.len <= 0 || !vdit::attn_uses_key_bound(p, key_norm_max > 0.f)) return VDIT_OK;
  if (key_norm_max > 0.f) {
    p.kbound_sq = key_norm_max * key_norm_max;
    return VDIT_OK;
  }
  if (!area) return VDIT_OK;
  float* out = reinterpret_cast<float*>(area);
  if (auto st = from_hip(vdit::launch_key_bound(keys, p.B, p.Hk, p.D, part_len, out, stream), "key bound launch");
      st != VDIT_OK)
    return st;
  p.kbound = out;
  p.kbound_n = vdit::kKeyBoundBlocks;
  return VDIT_OK;
}

// Plain attention of p (FULL or ROLLING), with the key-norm bound and the
// key split when the caller's workspace holds them (bound first, then the
// split partials); a missing or smaller workspace runs without them.
vdit_status launch_plain(vdit::AttnLaunch p, const vdit::AttnArgs& a, hipStream_t stream, const char* what) {
  const int64_t keys = p.nseg ? p.seg[0].len : 0;
  const size_t kb = vdit::kbound_bytes(a);
  char* bound = optional_area(a, 0, kb);
  const vdit::SplitPlan sp = vdit::split_plan(a.dtype, a.B, a.Lq, a.n_heads, keys, vdit::device_cus());
  const size_t need = vdit::split_workspace_bytes(sp, a.B, a.Lq, a.n_heads, a.head_dim);
  char* ws = optional_area(a, kb, need);
  if (ws) {
    p.nsplit = sp.nsplit;
    p.split_keys = sp.split_keys;
    p.epi = vdit::kEpiRing;  // every key range writes its float32 partial
    p.has_prev = 0;
    p.final_out = 0;
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(
        ws + vdit::align256(size_t(sp.nsplit) * size_t(a.B) * size_t(a.Lq) * size_t(a.n_heads) * size_t(a.head_dim) * 4));
  }
  if (p.nseg)
    if (auto st = add_key_bound(p, p.seg[0], bound, stream, a.key_norm_max); st != VDIT_OK) return st;
  if (auto st = from_hip(launch_attn(p, a.dtype, stream), what); st != VDIT_OK) return st;
  if (!ws) return VDIT_OK;
  vdit::SplitMergeLaunch m;
  m.part_o = p.part_o;
  m.part_lse = p.part_lse;
  m.o = a.o;
  m.lse = a.lse;
  m.L = a.Lq;
  m.B = a.B;
  m.H = a.n_heads;
  m.D = a.head_dim;
  m.nsplit = sp.nsplit;
  m.out_dtype = a.dtype;
  return from_hip(vdit::launch_split_merge(m, stream), what);
}

}  // namespace

namespace vdit {
// Records msg as the calling thread's vdit_last_error() and returns status
// (for entry points defined outside this file).
int report_error(int status, const char* msg) {
  g_last_error = msg;
  return status;
}
}  // namespace vdit

extern "C" {

const char* vdit_last_error(void) { return g_last_error.c_str(); }

int32_t vdit_abi_version(void) { return VDIT_ABI_VERSION; }

vdit_status vdit_rope_qkv(const void* q_in, const void* k_in, const void* v_in, void* q_out, void* k_out,
                          void* v_out, int32_t B, int64_t L, int32_t n_heads, int32_t n_kv_heads,
                          int32_t head_dim, vdit_dtype dtype, const vdit_grid* grid, int64_t token0,
                          int64_t t_offset, const float* q_gain, const float* k_gain, const float* v_gain,
                          float eps, uint32_t flags, hipStream_t stream) {
  static_assert(sizeof(vdit_grid) == sizeof(vdit::GridArgs), "vdit_grid layout mirror");
  const auto* g = reinterpret_cast<const vdit::GridArgs*>(grid);
  if (auto r = vdit::check_rope(q_in, k_in, q_out, k_out, B, L, n_heads, n_kv_heads, head_dim,
                                int(dtype), g, token0, eps, v_in, v_out);
      !r)
    return from_check(r);
  for (const float* gp : {q_gain, k_gain, v_gain})
    if (gp && (reinterpret_cast<uintptr_t>(gp) & 15)) return fail(VDIT_ERR_INVALID_ARG, "gain pointers must be 16-byte aligned");
  if (flags & ~uint32_t(VDIT_ROPE_NO_NORM | VDIT_ROPE_NO_Q_NORM | VDIT_ROPE_V_NORM))
    return fail(VDIT_ERR_INVALID_ARG, "unknown rope flags");
  vdit::RopeLaunch p;
  p.q_in = q_in;
  p.k_in = k_in;
  p.q_out = q_out;
  p.k_out = k_out;
  p.q_gain = q_gain;
  p.k_gain = k_gain;
  p.v_in = v_in;
  p.v_out = v_out;
  p.v_gain = v_gain;
  p.L = L;
  p.token0 = token0;
  p.t_offset = t_offset;
  p.B = B;
  p.Hq = n_heads;
  p.Hk = n_kv_heads;
  p.D = head_dim;
  p.T = g->T;
  p.H = g->H;
  p.W = g->W;
  p.pairs_t = g->pairs_t;
  p.pairs_h = g->pairs_h;
  p.pairs_w = g->pairs_w;
  p.theta = g->theta;
  p.eps = eps;
  p.norm_k = (flags & VDIT_ROPE_NO_NORM) ? 0 : 1;
  p.norm_q = (flags & (VDIT_ROPE_NO_NORM | VDIT_ROPE_NO_Q_NORM)) ? 0 : 1;
  p.norm_v = (flags & VDIT_ROPE_V_NORM) ? 1 : 0;
  p.dtype = int32_t(dtype);
  return from_hip(vdit::launch_rope(p, stream), "rope launch");
}

vdit_status vdit_rope_qk(const void* q_in, const void* k_in, void* q_out, void* k_out, int32_t B,
                         int64_t L, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                         vdit_dtype dtype, const vdit_grid* grid, int64_t token0, int64_t t_offset,
                         const float* q_gain, const float* k_gain, float eps, uint32_t flags,
                         hipStream_t stream) {
  if (flags & VDIT_ROPE_V_NORM) return fail(VDIT_ERR_INVALID_ARG, "VDIT_ROPE_V_NORM belongs to vdit_rope_qkv");
  return vdit_rope_qkv(q_in, k_in, nullptr, q_out, k_out, nullptr, B, L, n_heads, n_kv_heads, head_dim, dtype,
                       grid, token0, t_offset, q_gain, k_gain, nullptr, eps, flags, stream);
}

vdit_status vdit_rms_norm(const void* x_in, void* x_out, int32_t B, int64_t L, int32_t n_heads,
                          int32_t head_dim, vdit_dtype dtype, const float* gain, float eps,
                          hipStream_t stream) {
  if (auto r = vdit::check_rms_norm(x_in, x_out, B, L, n_heads, head_dim, int(dtype), gain, eps); !r)
    return from_check(r);
  vdit::RmsNormLaunch p;
  p.x_in = x_in;
  p.x_out = x_out;
  p.gain = gain;
  p.rows = int64_t(B) * L * n_heads;
  p.D = head_dim;
  p.eps = eps;
  p.dtype = int32_t(dtype);
  return from_hip(vdit::launch_rms_norm(p, stream), "vdit_rms_norm launch");
}

size_t vdit_attn_workspace_bytes(const vdit_attn_args* args) {
  if (!args) return size_t(-1);
  const vdit::AttnArgs& a = mirror(args);
  if (auto r = vdit::check_attn_shape(a); !r) {
    g_last_error = r.msg;
    return size_t(-1);
  }
  return vdit::attn_workspace_bytes(a, vdit::device_cus());
}

vdit_status vdit_attn_fwd(const vdit_attn_args* args, hipStream_t stream) {
  if (!args) return fail(VDIT_ERR_INVALID_ARG, "args is NULL");
  const vdit::AttnArgs& a = mirror(args);
  if (auto r = vdit::check_attn(a); !r) return from_check(r);
  const size_t es = vdit::esize(a.dtype);
  const int64_t D = a.head_dim;
  const bool empty_q = (a.B == 0 || a.Lq == 0);

  switch (a.mode) {
    case VDIT_ATTN_FULL: {
      if (empty_q) return VDIT_OK;
      vdit::AttnLaunch p = base_launch(a);
      if (a.Lkv > 0) {
        p.nseg = 1;
        p.seg[0] = {a.k, a.v, a.Lkv, a.Lkv * a.n_kv_heads * D};
      }
      return launch_plain(p, a, stream, "vdit_attn_fwd(FULL) launch");
    }
    case VDIT_ATTN_RING: {
      if (empty_q) return VDIT_OK;
      const int n = a.n_kv_chunks;
      auto seg_of = [&](int c) -> vdit::KvSeg {
        return {a.k_chunks[c], a.v_chunks[c], a.chunk_len[c], a.chunk_len[c] * a.n_kv_heads * D};
      };
      // workspace: [running partial (required)] [key bounds, one run per
      // chunk] [one float32 partial per chunk (one-launch form)]
      const size_t req = vdit::ring_workspace_bytes(a), kb = vdit::kbound_bytes(a);
      const size_t run_floats = size_t(a.B) * size_t(a.n_kv_heads) * vdit::kKeyBoundParts;
      char* bound = optional_area(a, req, kb);
      auto bound_run = [&](int c) -> char* { return bound ? bound + size_t(c) * run_floats * 4 : nullptr; };
      char* parts = optional_area(a, req + kb, vdit::ring_partials_bytes(a));
      if (parts) {
        // every chunk at once: split s of the launch attends to chunk s
        vdit::AttnLaunch p = base_launch(a);
        p.nseg = n;
        bool all_keys = true;
        for (int c = 0; c < n; ++c) {
          p.seg[c] = seg_of(c);
          all_keys = all_keys && a.chunk_len[c] > 0;
        }
        p.nsplit = n;
        p.seg_split = 1;
        p.epi = vdit::kEpiRing;  // each chunk writes its float32 partial
        p.has_prev = 0;
        p.final_out = 0;
        p.part_o = reinterpret_cast<float*>(parts);
        p.part_lse = reinterpret_cast<float*>(
            parts + vdit::align256(size_t(n) * size_t(a.B) * size_t(a.Lq) * size_t(a.n_heads) * size_t(D) * 4));
        if (a.key_norm_max > 0.f && all_keys && vdit::attn_uses_key_bound(p, true)) {
          p.kbound_sq = a.key_norm_max * a.key_norm_max;
        } else if (bound && all_keys && vdit::attn_uses_key_bound(p, false)) {
          for (int c = 0; c < n; ++c)
            if (auto st = from_hip(vdit::launch_key_bound(p.seg[c], p.B, p.Hk, p.D, 0,
                                                          reinterpret_cast<float*>(bound_run(c)), stream),
                                   "key bound launch");
                st != VDIT_OK)
              return st;
          p.kbound = reinterpret_cast<const float*>(bound);
          p.kbound_n = vdit::kKeyBoundBlocks;
        }
        if (auto st = from_hip(launch_attn(p, a.dtype, stream), "vdit_attn_fwd(RING) launch"); st != VDIT_OK)
          return st;
        vdit::SplitMergeLaunch m;
        m.part_o = p.part_o;
        m.part_lse = p.part_lse;
        m.o = a.o;
        m.lse = a.lse;
        m.L = a.Lq;
        m.B = a.B;
        m.H = a.n_heads;
        m.D = a.head_dim;
        m.nsplit = n;
        m.out_dtype = a.dtype;
        return from_hip(vdit::launch_split_merge(m, stream), "vdit_attn_fwd(RING) merge");
      }
      if (n == 1) {
        vdit::AttnLaunch p = base_launch(a);
        if (a.chunk_len[0] > 0) {
          p.nseg = 1;
          p.seg[0] = seg_of(0);
          if (auto st = add_key_bound(p, p.seg[0], bound, stream, a.key_norm_max); st != VDIT_OK) return st;
        }
        return from_hip(launch_attn(p, a.dtype, stream), "vdit_attn_fwd(RING) launch");
      }
      char* ws = static_cast<char*>(a.workspace);
      float* part_o = reinterpret_cast<float*>(ws);
      float* part_lse = reinterpret_cast<float*>(
          ws + vdit::align256(size_t(a.B) * size_t(a.Lq) * size_t(a.n_heads) * size_t(D) * 4));
      for (int c = 0; c < n; ++c) {
        vdit::AttnLaunch p = base_launch(a);
        if (a.chunk_len[c] > 0) {
          p.nseg = 1;
          p.seg[0] = seg_of(c);
          if (auto st = add_key_bound(p, p.seg[0], bound_run(c), stream, a.key_norm_max); st != VDIT_OK)
            return st;
        }
        p.epi = vdit::kEpiRing;
        p.part_o = part_o;
        p.part_lse = part_lse;
        p.has_prev = c > 0;
        p.final_out = c == n - 1;
        if (auto st = from_hip(launch_attn(p, a.dtype, stream), "vdit_attn_fwd(RING) launch"); st != VDIT_OK)
          return st;
      }
      return VDIT_OK;
    }
    case VDIT_ATTN_ROLLING: {
      if (empty_q) return VDIT_OK;
      // cache [B, n_slots, Lq, Hk, D]: frame f lives in slot f mod n_slots
      const size_t frame_elems = size_t(a.Lq) * size_t(a.n_kv_heads) * size_t(D);  // one batch, one slot
      const int64_t slot = a.frame % a.n_slots;
      char* kc = static_cast<char*>(a.k_cache);
      char* vc = static_cast<char*>(a.v_cache);
      const size_t pitch = size_t(a.n_slots) * frame_elems * es;
      for (int which = 0; which < 2; ++which) {
        const void* src = which ? a.v : a.k;
        char* dst = (which ? vc : kc) + size_t(slot) * frame_elems * es;
        if (!src || src == dst) continue;
        if (auto st = from_hip(hipMemcpy2DAsync(dst, pitch, src, frame_elems * es, frame_elems * es, size_t(a.B),
                                                hipMemcpyDeviceToDevice, stream),
                               "vdit_attn_fwd(ROLLING) cache insert");
            st != VDIT_OK)
          return st;
      }
      // Frames 0..frame sit in slots 0..frame until the ring is full, after
      // which every slot is valid: the valid keys of each batch are always
      // the contiguous prefix of min(frame + 1, n_slots) slots.  Softmax
      // attention does not depend on key order, so they are one segment.
      const int64_t nvalid = a.frame + 1 < a.n_slots ? a.frame + 1 : a.n_slots;
      vdit::AttnLaunch p = base_launch(a);
      p.nseg = 1;
      p.seg[0] = {kc, vc, nvalid * a.Lq, int64_t(a.n_slots) * a.Lq * a.n_kv_heads * D};
      return launch_plain(p, a, stream, "vdit_attn_fwd(ROLLING) launch");
    }
    case VDIT_ATTN_CHUNK_HYBRID: {
      const vdit::HybridLayout lay = vdit::hybrid_layout(a);
      char* ws = static_cast<char*>(a.workspace);
      vdit::HybridStateLaunch hs;
      std::memset(&hs, 0, sizeof(hs));
      hs.k = a.k;
      hs.v = a.v;
      hs.s_in = a.state_s;
      hs.z_in = a.state_z;
      hs.zero_in = (a.flags & vdit::kAttnStateZero) ? 1 : 0;
      hs.s_out = a.state_s;
      hs.z_out = a.state_z;
      hs.ds = reinterpret_cast<float*>(ws + lay.off_ds);
      hs.dz = reinterpret_cast<float*>(ws + lay.off_dz);
      hs.sc = ws + lay.off_sc;
      hs.zc = reinterpret_cast<float*>(ws + lay.off_zc);
      hs.L = a.Lq;
      hs.Lkv = a.Lkv;
      hs.ctx = a.ctx_tokens;
      hs.overlap = a.overlap_tokens;
      hs.chunk = a.chunk_tokens;
      hs.n_chunks = lay.n_chunks;
      hs.nsplit = lay.nsplit;
      hs.B = a.B;
      hs.Hk = a.n_kv_heads;
      hs.D = a.head_dim;
      hs.dtype = a.dtype;
      const vdit::FeatureMap fq = feature_map(a.phi_coef, 0), fk = feature_map(a.phi_coef, 4);
      hs.phi_k = fk;
      if (auto st = from_hip(vdit::launch_hybrid_state(hs, stream), "vdit_attn_fwd(CHUNK_HYBRID) state");
          st != VDIT_OK)
        return st;
      if (empty_q) return VDIT_OK;
      vdit::AttnLaunch p = base_launch(a);
      p.epi = vdit::kEpiHybrid;
      p.chunk = a.chunk_tokens;
      p.n_chunks = lay.n_chunks;
      p.hyb_ctx = a.ctx_tokens;
      p.hyb_overlap = a.overlap_tokens;
      p.hyb_lkv = a.Lkv;
      p.st = ws + lay.off_sc;
      p.zc = reinterpret_cast<const float*>(ws + lay.off_zc);
      p.hk = a.k;
      p.hv = a.v;
      p.phi_q = fq;
      p.nseg = 1;
      char* bound = optional_area(a, lay.total, vdit::kbound_bytes(a));
      // a bound per chunk (so a chunk's result does not depend on the others);
      // overlapping windows run on the online maximum unless the caller gives
      // a bound for every key
      if (a.overlap_tokens == 0 || a.key_norm_max > 0.f)
        if (auto st = add_key_bound(p, vdit::KvSeg{a.k, a.v, a.Lq, a.Lq * a.n_kv_heads * D}, bound, stream,
                                    a.key_norm_max, a.chunk_tokens);
            st != VDIT_OK)
          return st;
      return from_hip(launch_attn(p, a.dtype, stream), "vdit_attn_fwd(CHUNK_HYBRID) launch");
    }
  }
  return fail(VDIT_ERR_INVALID_ARG, "unknown attention mode");
}

vdit_status vdit_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                           void* o_out, float* lse_out, vdit_dtype in_dtype, vdit_dtype out_dtype,
                           int32_t B, int64_t L, int32_t n_heads, int32_t head_dim,
                           hipStream_t stream) {
  if (auto r = vdit::check_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out, int(in_dtype),
                                 int(out_dtype), B, L, n_heads, head_dim);
      !r)
    return from_check(r);
  vdit::MergeLaunch p;
  p.o_a = o_a;
  p.lse_a = lse_a;
  p.o_b = o_b;
  p.lse_b = lse_b;
  p.o_out = o_out;
  p.lse_out = lse_out;
  p.L = L;
  p.B = B;
  p.H = n_heads;
  p.D = head_dim;
  p.in_dtype = int32_t(in_dtype);
  p.out_dtype = int32_t(out_dtype);
  return from_hip(vdit::launch_merge(p, stream), "vdit_lse_merge launch");
}

}  // extern "C"
