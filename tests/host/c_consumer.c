/* A plain C consumer of libvdit: device buffers from hipMalloc, a stream of
 * its own, workspace sized by vdit_attn_workspace_bytes, statuses checked.
 * No Python and no torch: it exercises the C ABI of include/vdit.h as a C
 * program would.
 *
 *   c_consumer <dir>
 *
 * Reads <dir>/meta.txt ("L Hq Hk D T H W pairs_t pairs_h pairs_w split"),
 * <dir>/q.bin, k.bin, v.bin (bfloat16 bit patterns, [1, L, H, D]); runs
 * RMSNorm + 3D-RoPE of q and k (vdit_rope_qk, and vdit_rope_qkv with the
 * values normalised in the same launch, whose q and k must equal the first
 * call's bit for bit), FULL attention, and RING attention over the two key
 * chunks [0, split) and [split, L); writes qr.bin, kr.bin, vn.bin (bf16),
 * o_full.bin, o_ring.bin (bf16), lse_full.bin, lse_ring.bin (float32).  It
 * also checks that an unsupported head dimension is refused with a message.
 * Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "vdit.h"

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));       \
      return 1;                                                            \
    }                                                                      \
  } while (0)

#define VDIT_OK_(x)                                                        \
  do {                                                                     \
    vdit_status s_ = (x);                                                  \
    if (s_ != VDIT_OK) {                                                   \
      fprintf(stderr, "%s: status %d: %s\n", #x, (int)s_, vdit_last_error()); \
      return 1;                                                            \
    }                                                                      \
  } while (0)

static int read_file(const char* dir, const char* name, void* dst, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return 1;
  size_t got = fread(dst, 1, n, f);
  fclose(f);
  return got == n ? 0 : 1;
}

static int write_file(const char* dir, const char* name, const void* src, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = fwrite(src, 1, n, f);
  fclose(f);
  return put == n ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <dir>\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/meta.txt", dir);
  FILE* mf = fopen(path, "r");
  if (!mf) {
    fprintf(stderr, "cannot open %s\n", path);
    return 1;
  }
  long L, split;
  int Hq, Hk, D, T, H, W, pt, ph, pw;
  int nread = fscanf(mf, "%ld %d %d %d %d %d %d %d %d %d %ld", &L, &Hq, &Hk, &D, &T, &H, &W, &pt, &ph, &pw, &split);
  fclose(mf);
  if (nread != 11 || L <= 0 || split <= 0 || split >= L) {
    fprintf(stderr, "bad meta.txt\n");
    return 1;
  }
  if (vdit_abi_version() != VDIT_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", vdit_abi_version(), VDIT_ABI_VERSION);
    return 1;
  }
  const size_t nq = (size_t)L * Hq * D, nk = (size_t)L * Hk * D, nl = (size_t)Hq * L;
  uint16_t* hq = (uint16_t*)malloc(nq * 2);
  uint16_t* hk = (uint16_t*)malloc(nk * 2);
  uint16_t* hv = (uint16_t*)malloc(nk * 2);
  uint16_t* ho = (uint16_t*)malloc(nq * 2);
  float* hl = (float*)malloc(nl * 4);
  if (!hq || !hk || !hv || !ho || !hl) return 1;
  if (read_file(dir, "q.bin", hq, nq * 2) || read_file(dir, "k.bin", hk, nk * 2) || read_file(dir, "v.bin", hv, nk * 2)) {
    fprintf(stderr, "cannot read inputs\n");
    return 1;
  }

  void *q, *k, *v, *qr, *kr, *o_full, *o_ring;
  float *lse_full, *lse_ring;
  HIP_OK(hipMalloc(&q, nq * 2));
  HIP_OK(hipMalloc(&k, nk * 2));
  HIP_OK(hipMalloc(&v, nk * 2));
  HIP_OK(hipMalloc(&qr, nq * 2));
  HIP_OK(hipMalloc(&kr, nk * 2));
  HIP_OK(hipMalloc(&o_full, nq * 2));
  HIP_OK(hipMalloc(&o_ring, nq * 2));
  HIP_OK(hipMalloc((void**)&lse_full, nl * 4));
  HIP_OK(hipMalloc((void**)&lse_ring, nl * 4));
  HIP_OK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, nk * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, nk * 2, hipMemcpyHostToDevice));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  /* RMSNorm + 3D-RoPE */
  vdit_grid g = {T, H, W, pt, ph, pw, 10000.0f};
  VDIT_OK_(vdit_rope_qk(q, k, qr, kr, 1, L, Hq, Hk, D, VDIT_BF16, &g, 0, 0, NULL, NULL, 1e-6f, 0u, s));
  /* the same, with the values normalised in the same launch */
  void *q2, *k2, *vn;
  HIP_OK(hipMalloc(&q2, nq * 2));
  HIP_OK(hipMalloc(&k2, nk * 2));
  HIP_OK(hipMalloc(&vn, nk * 2));
  VDIT_OK_(vdit_rope_qkv(q, k, v, q2, k2, vn, 1, L, Hq, Hk, D, VDIT_BF16, &g, 0, 0, NULL, NULL, NULL, 1e-6f,
                         VDIT_ROPE_V_NORM, s));

  /* FULL */
  vdit_attn_args a;
  memset(&a, 0, sizeof a);
  a.mode = VDIT_ATTN_FULL;
  a.dtype = VDIT_BF16;
  a.B = 1;
  a.n_heads = Hq;
  a.n_kv_heads = Hk;
  a.head_dim = D;
  a.Lq = L;
  a.Lkv = L;
  a.q = qr;
  a.k = kr;
  a.v = v;
  a.o = o_full;
  a.lse = lse_full;
  size_t ws_full = vdit_attn_workspace_bytes(&a);
  if (ws_full == (size_t)-1) {
    fprintf(stderr, "workspace query failed: %s\n", vdit_last_error());
    return 1;
  }
  void* ws1 = NULL;
  if (ws_full) HIP_OK(hipMalloc(&ws1, ws_full));
  a.workspace = ws1;
  a.workspace_bytes = ws_full;
  VDIT_OK_(vdit_attn_fwd(&a, s));

  /* RING over two key chunks of the rotated keys */
  const void* kc[2] = {kr, (const char*)kr + (size_t)split * Hk * D * 2};
  const void* vc[2] = {v, (const char*)v + (size_t)split * Hk * D * 2};
  int64_t lens[2] = {split, L - split};
  vdit_attn_args r = a;
  r.mode = VDIT_ATTN_RING;
  r.k = NULL;
  r.v = NULL;
  r.o = o_ring;
  r.lse = lse_ring;
  r.n_kv_chunks = 2;
  r.k_chunks = kc;
  r.v_chunks = vc;
  r.chunk_len = lens;
  r.workspace = NULL;
  r.workspace_bytes = 0;
  size_t ws_ring = vdit_attn_workspace_bytes(&r);
  if (ws_ring == (size_t)-1 || ws_ring == 0) {
    fprintf(stderr, "ring workspace query: %s\n", vdit_last_error());
    return 1;
  }
  void* ws2 = NULL;
  HIP_OK(hipMalloc(&ws2, ws_ring));
  r.workspace = ws2;
  r.workspace_bytes = ws_ring;
  VDIT_OK_(vdit_attn_fwd(&r, s));

  /* an unsupported head dimension is refused before any launch */
  vdit_attn_args bad = a;
  bad.head_dim = 96;
  if (vdit_attn_fwd(&bad, s) != VDIT_ERR_UNSUPPORTED || strlen(vdit_last_error()) == 0) {
    fprintf(stderr, "head_dim 96 was not refused\n");
    return 1;
  }

  HIP_OK(hipStreamSynchronize(s));
  /* vdit_rope_qkv's q and k are vdit_rope_qk's, bit for bit */
  {
    void* h1 = malloc(nq * 2);
    void* h2 = malloc(nq * 2);
    if (!h1 || !h2) {
      fprintf(stderr, "out of host memory\n");
      return 1;
    }
    HIP_OK(hipMemcpy(h1, qr, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h2, q2, nq * 2, hipMemcpyDeviceToHost));
    int differ = memcmp(h1, h2, nq * 2) != 0;
    HIP_OK(hipMemcpy(h1, kr, nk * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h2, k2, nk * 2, hipMemcpyDeviceToHost));
    differ |= memcmp(h1, h2, nk * 2) != 0;
    free(h1);
    free(h2);
    if (differ) {
      fprintf(stderr, "vdit_rope_qkv's q or k differ from vdit_rope_qk's\n");
      return 1;
    }
  }
  int bad_io = 0;
  HIP_OK(hipMemcpy(ho, qr, nq * 2, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "qr.bin", ho, nq * 2);
  HIP_OK(hipMemcpy(hk, kr, nk * 2, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "kr.bin", hk, nk * 2);
  HIP_OK(hipMemcpy(ho, o_full, nq * 2, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "o_full.bin", ho, nq * 2);
  HIP_OK(hipMemcpy(hl, lse_full, nl * 4, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "lse_full.bin", hl, nl * 4);
  HIP_OK(hipMemcpy(ho, o_ring, nq * 2, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "o_ring.bin", ho, nq * 2);
  HIP_OK(hipMemcpy(hl, lse_ring, nl * 4, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "lse_ring.bin", hl, nl * 4);
  HIP_OK(hipMemcpy(hk, vn, nk * 2, hipMemcpyDeviceToHost));
  bad_io |= write_file(dir, "vn.bin", hk, nk * 2);
  if (bad_io) {
    fprintf(stderr, "cannot write outputs\n");
    return 1;
  }

  HIP_OK(hipStreamDestroy(s));
  void* bufs[] = {q, k, v, qr, kr, o_full, o_ring, lse_full, lse_ring, ws1, ws2, q2, k2, vn};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  free(hq);
  free(hk);
  free(hv);
  free(ho);
  free(hl);
  printf("c_consumer ok\n");
  return 0;
}
