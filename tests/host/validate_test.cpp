// Host-only test of the argument validation in validate.hpp (no HIP calls).
// Built with g++ (optionally under AddressSanitizer / UBSan) by the CPU tests.
#include <cstdio>
#include <cstdlib>
#include <string>

#include "validate.hpp"

using namespace vdit;

static int failures = 0;
#define EXPECT(cond, what)                                   \
  do {                                                       \
    if (!(cond)) {                                           \
      std::printf("FAIL %s (line %d)\n", what, __LINE__);    \
      ++failures;                                            \
    }                                                        \
  } while (0)

static void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }

int main() {
  GridArgs g{21, 30, 52, 22, 21, 21, 10000.f};
  // good rope call
  EXPECT(bool(check_rope(P(1ull << 30), P(2ull << 30), P(1ull << 30), P(2ull << 30), 1, 32760, 12, 12, 128, 0, &g, 0, 1e-6f)), "rope ok");
  EXPECT(check_rope(P(0x1000), nullptr, P(0x1000), nullptr, 1, 10, 12, 12, 96, 0, &g, 0, 1e-6f).code == Check::unsupported, "head_dim 96 unsupported");
  GridArgs bad = g; bad.pairs_w = 20;
  EXPECT(check_rope(P(0x1000), nullptr, P(0x1000), nullptr, 1, 10, 12, 12, 128, 0, &bad, 0, 1e-6f).code == Check::invalid, "pair sum");
  EXPECT(check_rope(P(0x1000), nullptr, P(0x1000), nullptr, 1, 10, 12, 12, 128, 0, nullptr, 0, 1e-6f).code == Check::invalid, "null grid");
  EXPECT(check_rope(P(0x1001), nullptr, P(0x1001), nullptr, 1, 10, 12, 12, 128, 0, &g, 0, 1e-6f).code == Check::invalid, "alignment");
  EXPECT(check_rope(P(0x1000), nullptr, P(0x1000), nullptr, 1, 32761, 12, 12, 128, 0, &g, 0, 1e-6f).code == Check::invalid, "beyond grid");
  EXPECT(check_rope(P(0x1000), nullptr, P(0x1010), nullptr, 1, 10, 12, 12, 128, 0, &g, 0, 1e-6f).code == Check::invalid, "partial overlap");
  EXPECT(check_rope(P(0x1000), nullptr, nullptr, nullptr, 1, 10, 12, 12, 128, 0, &g, 0, 1e-6f).code == Check::invalid, "q_out missing");
  EXPECT(check_rope(P(0x1000), nullptr, P(0x1000), nullptr, 1, 10, 12, 12, 128, 0, &g, 0, -1.f).code == Check::invalid, "negative eps");
  // the values of vdit_rope_qkv (q, k at 1 GiB, 2 GiB; v at 3 GiB; one tensor is 1 x 32760 x 12 x 128 bf16)
  EXPECT(bool(check_rope(P(1ull << 30), P(2ull << 30), P(1ull << 30), P(2ull << 30), 1, 32760, 12, 12, 128, 0, &g, 0,
                         1e-6f, P(3ull << 30), P(3ull << 30))), "rope with values in place ok");
  EXPECT(check_rope(P(1ull << 30), P(2ull << 30), P(1ull << 30), P(2ull << 30), 1, 32760, 12, 12, 128, 0, &g, 0,
                    1e-6f, P(3ull << 30), nullptr).code == Check::invalid, "v_out missing");
  EXPECT(check_rope(P(1ull << 30), P(2ull << 30), P(1ull << 30), P(2ull << 30), 1, 32760, 12, 12, 128, 0, &g, 0,
                    1e-6f, P(3ull << 30), P((2ull << 30) + 4096)).code == Check::invalid, "v_out over k_out");
  EXPECT(check_rope(P(1ull << 30), P(2ull << 30), P(1ull << 30), P((3ull << 30) + 64), 1, 32760, 12, 12, 128, 0, &g,
                    0, 1e-6f, P(3ull << 30), P(4ull << 30)).code == Check::invalid, "k_out over v_in");
  EXPECT(check_rope(P(1ull << 30), P(2ull << 30), P(1ull << 30), P(2ull << 30), 1, 10, 64, 64, 128, 0, &g, 0, 1e-6f,
                    P(3ull << 30), P(3ull << 30)).code == Check::unsupported, "too many rows per token with values");

  // per-head RMSNorm (values of KV-norm attention)
  EXPECT(bool(check_rms_norm(P(0x1000), P(0x1000), 1, 3600, 3, 64, 0, nullptr, 1e-6f)), "rms norm in place ok");
  EXPECT(bool(check_rms_norm(P(0x1000), P(1ull << 24), 1, 3600, 3, 64, 0, nullptr, 1e-6f)), "rms norm out of place ok");
  EXPECT(check_rms_norm(P(0x1000), P(0x1010), 1, 10, 3, 64, 0, nullptr, 1e-6f).code == Check::invalid, "rms norm partial overlap");
  EXPECT(check_rms_norm(P(0x1000), P(0x1000), 1, 10, 3, 256, 0, nullptr, 1e-6f).code == Check::unsupported, "rms norm head_dim");
  EXPECT(check_rms_norm(P(0x1000), nullptr, 1, 10, 3, 64, 0, nullptr, 1e-6f).code == Check::invalid, "rms norm out missing");
  EXPECT(bool(check_rms_norm(nullptr, nullptr, 1, 0, 3, 64, 0, nullptr, 1e-6f)), "rms norm empty with NULL");
  EXPECT(check_rms_norm(P(0x1000), P(0x1000), 1, 10, 3, 64, 0, (const float*)P(0x2004), 1e-6f).code == Check::invalid, "rms norm gain alignment");
  EXPECT(check_rms_norm(P(0x1000), P(0x1000), 1, 10, 3, 64, 2, nullptr, 1e-6f).code == Check::invalid, "rms norm dtype");

  AttnArgs a{};
  a.mode = 0; a.dtype = 0; a.B = 1; a.n_heads = 12; a.n_kv_heads = 12; a.head_dim = 128;
  a.Lq = 100; a.Lkv = 100; a.q = P(1ull << 28); a.k = P(2ull << 28); a.v = P(3ull << 28); a.o = P(4ull << 28);
  EXPECT(bool(check_attn(a)), "full ok");
  AttnArgs b = a; b.n_kv_heads = 5;
  EXPECT(check_attn(b).code == Check::invalid, "heads divisibility");
  b = a; b.o = P((1ull << 28) + 0x100);
  EXPECT(check_attn(b).code == Check::invalid, "o aliases q");
  b = a; b.head_dim = 256;
  EXPECT(check_attn(b).code == Check::unsupported, "head_dim 256");
  b = a; b.mode = 7;
  EXPECT(check_attn(b).code == Check::invalid, "mode");

  // ring
  const void* kc[2] = {P(5ull << 28), P(6ull << 28)};
  const void* vc[2] = {P(7ull << 28), P(8ull << 28)};
  int64_t lens[2] = {60, 40};
  b = a; b.mode = 1; b.n_kv_chunks = 2; b.k_chunks = kc; b.v_chunks = vc; b.chunk_len = lens;
  EXPECT(check_attn(b).code == Check::invalid, "ring workspace missing");
  b.workspace = P(9ull << 28); b.workspace_bytes = ring_workspace_bytes(b);
  EXPECT(bool(check_attn(b)), "ring ok");
  lens[1] = 41;
  EXPECT(check_attn(b).code == Check::invalid, "ring lengths must sum to Lkv");
  lens[1] = 40;
  b.workspace_bytes -= 1;
  EXPECT(check_attn(b).code == Check::invalid, "ring workspace too small");

  // rolling
  b = a; b.mode = 2; b.n_slots = 5; b.frame = 3; b.k_cache = P(10ull << 28); b.v_cache = P(11ull << 28);
  EXPECT(bool(check_attn(b)), "rolling ok");
  b.n_slots = 0;
  EXPECT(check_attn(b).code == Check::invalid, "rolling slots");
  b.n_slots = 64;
  EXPECT(bool(check_attn(b)), "rolling many slots");
  b.n_slots = 5; b.frame = -1;
  EXPECT(check_attn(b).code == Check::invalid, "rolling frame");
  b.frame = 0; b.k = nullptr;
  EXPECT(check_attn(b).code == Check::invalid, "rolling k/v pairing");

  // hybrid
  b = a; b.mode = 3; b.chunk_tokens = 30; b.state_s = reinterpret_cast<float*>(P(12ull << 28));
  b.state_z = reinterpret_cast<float*>(P(13ull << 28));
  EXPECT(check_attn(b).code == Check::invalid, "hybrid workspace missing");
  b.workspace = P(14ull << 28); b.workspace_bytes = hybrid_layout(b).total;
  EXPECT(bool(check_attn(b)), "hybrid ok");
  HybridLayout hl = hybrid_layout(b);
  EXPECT(hl.n_chunks == 4, "hybrid chunk count");
  b.Lkv = 99;
  EXPECT(check_attn(b).code == Check::invalid, "hybrid Lkv");
  b.Lkv = 100; b.chunk_tokens = 0;
  EXPECT(check_attn(b).code == Check::invalid, "hybrid chunk");
  b.chunk_tokens = 30; b.overlap_tokens = 15; b.ctx_tokens = 15; b.Lkv = 115;
  EXPECT(bool(check_attn(b)), "hybrid with overlap and context");
  b.Lkv = 100;
  EXPECT(check_attn(b).code == Check::invalid, "hybrid Lkv = ctx + Lq");
  b.Lkv = 116; b.ctx_tokens = 16;
  EXPECT(check_attn(b).code == Check::invalid, "hybrid context beyond the overlap");
  b.ctx_tokens = 0; b.Lkv = 100; b.overlap_tokens = -1;
  EXPECT(check_attn(b).code == Check::invalid, "hybrid negative overlap");
  AttnArgs f = a; f.overlap_tokens = 4;
  EXPECT(check_attn(f).code == Check::invalid, "overlap outside the hybrid mode");

  // placement: every range a call writes (o, lse, workspace, caches, state)
  // overlaps none of its other tensors, checked before anything is enqueued
  {
    AttnArgs r = a; r.mode = 2; r.n_slots = 5; r.frame = 3; r.k_cache = P(10ull << 28); r.v_cache = P(11ull << 28);
    r.workspace = P((10ull << 28) + 4096); r.workspace_bytes = 1 << 20;  // inside k_cache
    EXPECT(check_attn(r).code == Check::invalid, "rolling: workspace overlaps the cache");
    r.workspace = P(15ull << 28);
    EXPECT(bool(check_attn(r)), "rolling: separate workspace");
    r.workspace = P((15ull << 28) + 8);
    EXPECT(check_attn(r).code == Check::invalid, "rolling: misaligned workspace");
    r.workspace = nullptr; r.workspace_bytes = 0;
    // the new frame may be the cache slot itself (B = 1) ...
    const size_t frame_bytes = size_t(r.Lq) * r.n_kv_heads * r.head_dim * 2;
    r.k = P((10ull << 28) + 3 * frame_bytes); r.v = P((11ull << 28) + 3 * frame_bytes);
    EXPECT(bool(check_attn(r)), "rolling: frame given as its own slot (B = 1)");
    // ... but not another part of the cache, nor the slot when B > 1
    r.k = P((10ull << 28) + 2 * frame_bytes);
    EXPECT(check_attn(r).code == Check::invalid, "rolling: frame inside another slot");
    r.k = P((10ull << 28) + 3 * frame_bytes); r.B = 2;
    r.k_cache = P(10ull << 28); r.v_cache = P(12ull << 28); r.v = P((12ull << 28) + 3 * frame_bytes);
    EXPECT(check_attn(r).code == Check::invalid, "rolling: slot alias with B = 2");
    r = a; r.mode = 2; r.n_slots = 5; r.frame = 3; r.k_cache = P(10ull << 28); r.v_cache = P(11ull << 28);
    r.k = P(16ull << 28); r.v = P(17ull << 28); r.lse = reinterpret_cast<float*>(P((16ull << 28) + 256));
    EXPECT(check_attn(r).code == Check::invalid, "rolling: lse overlaps the new keys");

    AttnArgs h = a; h.mode = 3; h.chunk_tokens = 30;
    h.state_s = reinterpret_cast<float*>(P(12ull << 28)); h.state_z = reinterpret_cast<float*>(P(13ull << 28));
    h.workspace = P((12ull << 28) + 1024); h.workspace_bytes = hybrid_layout(h).total;
    EXPECT(check_attn(h).code == Check::invalid, "hybrid: workspace overlaps the state");
    h.workspace = P(14ull << 28); h.workspace_bytes = hybrid_layout(h).total + (1 << 20);
    EXPECT(bool(check_attn(h)), "hybrid: separate, larger workspace");
    h.state_z = reinterpret_cast<float*>(P((2ull << 28) + 512));  // inside k
    EXPECT(check_attn(h).code == Check::invalid, "hybrid: state overlaps k");
    h.state_z = reinterpret_cast<float*>(P((12ull << 28) + 4096));  // inside state_s
    EXPECT(check_attn(h).code == Check::invalid, "hybrid: state_z overlaps state_s");
    h.state_z = reinterpret_cast<float*>(P(13ull << 28));
    h.workspace_bytes = hybrid_layout(h).total + (1ull << 28) + 1;  // reaches o
    h.o = P(15ull << 28);
    EXPECT(check_attn(h).code == Check::invalid, "hybrid: workspace reaches o");

    AttnArgs f = a; f.lse = reinterpret_cast<float*>(P((3ull << 28) + 64));
    EXPECT(check_attn(f).code == Check::invalid, "full: lse overlaps v");
    f.lse = nullptr; f.k = f.v = f.q;  // read-only tensors may alias each other
    EXPECT(bool(check_attn(f)), "full: q, k, v the same tensor");
  }

  // key split plan (256 compute units)
  {
    SplitPlan sp = split_plan(0, 1, 2040, 16, 5 * 2040, 256);  // rolling decode frame: 256 workgroups of 128 queries
    EXPECT(sp.nsplit == 2 && sp.split_keys == 5120, "rolling split in two");
    EXPECT(split_workspace_bytes(sp, 1, 2040, 16, 64) == align256(2ull * 2040 * 16 * 64 * 4) + align256(2ull * 16 * 2040 * 4), "split workspace");
    EXPECT(split_plan(0, 1, 32760, 12, 32760, 256).nsplit == 1, "large layer unsplit");
    EXPECT(split_plan(1, 1, 2040, 16, 10200, 256).nsplit == 1, "float32 unsplit");
    EXPECT(split_plan(0, 1, 300, 4, 333, 256).nsplit == 1, "too few keys to split");
    sp = split_plan(0, 1, 1000, 2, 5000, 256);  // 16 workgroups: up to 8 ranges of >= 256 keys
    EXPECT(sp.nsplit == 8 && sp.split_keys == 640, "eight ranges, last one ragged");
    EXPECT((sp.nsplit - 1) * sp.split_keys < 5000 && sp.nsplit * sp.split_keys >= 5000, "ranges cover the keys");
    AttnArgs r = a; r.mode = 2; r.n_slots = 5; r.frame = 0; r.Lq = 2040; r.n_heads = 16; r.n_kv_heads = 16; r.head_dim = 64;
    EXPECT(attn_keys(r) == 2040, "rolling keys at frame 0");
    r.frame = 9;
    EXPECT(attn_keys(r) == 5 * 2040, "rolling keys once the ring is full");
    EXPECT(attn_workspace_bytes(r, 256) == kbound_bytes(r) + split_workspace_bytes(split_plan(0, 1, 2040, 16, 10200, 256), 1, 2040, 16, 64), "rolling workspace");
    EXPECT(kbound_bytes(r) == 4096, "key-norm partials: 64 per (batch, kv head)");
    r.dtype = 1;
    EXPECT(kbound_bytes(r) == 0 && attn_workspace_bytes(r, 256) == 0, "float32 needs no optional workspace");
  }

  // merge
  EXPECT(bool(check_merge(P(0x1000), (float*)P(0x2000), P(0x3000), (float*)P(0x4000), P(0x1000), (float*)P(0x2000), 0, 0, 1, 8, 2, 64)), "merge in place ok");
  EXPECT(check_merge(P(0x1000), (float*)P(0x2000), P(0x3000), (float*)P(0x4000), P(0x1000), nullptr, 0, 1, 1, 8, 2, 64).code == Check::invalid, "merge in place dtype");
  EXPECT(check_merge(P(0x1000), (float*)P(0x2000), P(0x3000), (float*)P(0x4000), P(0x1010), nullptr, 0, 0, 1, 8, 2, 64).code == Check::invalid, "merge partial overlap");

  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("validate_test ok\n");
  return 0;
}
