/*
 * vdit.h -- C ABI of a gfx950 (MI355X) library for the attention layer of
 * Wan-style video diffusion transformers: per-head RMS-normalised queries and
 * keys with channel-split 3D rotary position embedding, and exact multi-head
 * softmax attention over a flattened T x H x W latent grid in four modes.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer unless marked (host).  The
 *    caller owns all memory; the library never allocates or frees device
 *    memory and keeps no global mutable state (thread-safe).
 *  - Calls are asynchronous: they validate their arguments, enqueue kernels
 *    on `stream` and return without synchronising.  A status of VDIT_OK
 *    means "enqueued".
 *  - Validation happens before any launch; a call that fails validation
 *    writes nothing.  VDIT_ERR_INVALID_ARG: malformed arguments;
 *    VDIT_ERR_UNSUPPORTED: well-formed but outside what the kernels handle
 *    (for example head_dim other than 64 or 128); VDIT_ERR_HIP: a HIP call
 *    or launch failed.  vdit_last_error() returns a message for the last
 *    non-OK status of the calling thread.
 *  - Tensors are row-major: q, k, v, o are [B, L, H, D] (D fastest);
 *    log-sum-exp is [B, H, L] float32, natural log; an empty key set gives
 *    LSE = -inf and O = 0.
 *  - Device buffers must be 16-byte aligned.
 *  - Element types: VDIT_BF16 (bfloat16, results rounded to nearest even) or
 *    VDIT_F32.  Internal arithmetic is float32 in both cases.
 */
#ifndef VDIT_H
#define VDIT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 5: vdit_rope_qkv and VDIT_ROPE_V_NORM added (the earlier entry points and
 * structs unchanged) */
#define VDIT_ABI_VERSION 5

typedef enum {
  VDIT_OK = 0,
  VDIT_ERR_INVALID_ARG = 1,
  VDIT_ERR_UNSUPPORTED = 2,
  VDIT_ERR_HIP = 3
} vdit_status;

typedef enum { VDIT_BF16 = 0, VDIT_F32 = 1 } vdit_dtype;

/*
 * Latent grid and rotary split.  Tokens are flattened t-major, then h, then
 * w (FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
 * Transformers, Sec. 3.1 writes latents as T' x H' x W').  The D/2 adjacent
 * channel pairs (2p, 2p+1) are split in order into pairs_t, pairs_h, pairs_w
 * pairs that rotate with the token's t, h and w coordinate respectively
 * (3D-RoPE applied separately to the temporal and spatial axes, FlashDecoder
 * Sec. 3.2 "Base Architecture").  Inside an axis block of P_a pairs, pair j
 * has angular frequency theta^(-j / P_a) (RoFormer's 1D frequencies for a
 * block of dimension 2 P_a).  pairs_t + pairs_h + pairs_w must equal
 * head_dim / 2.
 */
typedef struct {
  int32_t T, H, W;
  int32_t pairs_t, pairs_h, pairs_w;
  float theta; /* RoPE base, e.g. 10000 */
} vdit_grid;

/* vdit_rope_qk flags */
#define VDIT_ROPE_NO_NORM 1u   /* skip the RMSNorm of q and k, rotate only */
#define VDIT_ROPE_NO_Q_NORM 2u /* skip it for q only: k is normalised, q rotated
                                  only (KV-norm; normalise v with vdit_rms_norm,
                                  or in the same launch with vdit_rope_qkv) */
#define VDIT_ROPE_V_NORM 4u    /* vdit_rope_qkv only: RMS-normalise the values
                                  (with v_gain) instead of copying them */

/*
 * vdit_rope_qk -- fused per-head RMSNorm + 3D-RoPE of queries and keys.
 *
 * For every token i of the slice, every head and both q and k:
 *   y = x / sqrt(mean_d(x_d^2) + eps) * gain        (RMSNorm over head_dim,
 *       Zhang & Sennrich, cited by FlashDecoder Sec. 3.2; skipped with
 *       VDIT_ROPE_NO_NORM, and for q alone with VDIT_ROPE_NO_Q_NORM)
 *   then each pair (y_2p, y_2p+1) is rotated by angle alpha = pos * omega_p:
 *   (y0 cos a - y1 sin a, y0 sin a + y1 cos a).
 * Token i has grid index n = token0 + i, so t = n / (H W) + t_offset,
 * h = (n / W) mod H, w = n mod W.  t_offset lets a caller place a frame of a
 * stream at any temporal position (FlashDecoder Sec. 4 "Long Video
 * Decoding" assigns positions relative to the current window); angles are
 * reduced in float64 so large positions keep full float32 accuracy.
 *
 * q_in, q_out: [B, L, n_heads, head_dim]; k_in, k_out: [B, L, n_kv_heads,
 * head_dim]; dtype of all four.  q_out may equal q_in and k_out may equal
 * k_in (in place); partial overlap is not allowed.  k_in/k_out may both be
 * NULL (queries only) and likewise q_in/q_out.  q_gain, k_gain: [head_dim]
 * float32 or NULL (gain 1).  eps >= 0.  grid (host) is read during the
 * call only.  head_dim in {64, 128}; token0 + L <= T*H*W.
 */
vdit_status vdit_rope_qk(const void* q_in, const void* k_in, void* q_out, void* k_out,
                         int32_t B, int64_t L, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, vdit_dtype dtype, const vdit_grid* grid,
                         int64_t token0, int64_t t_offset, const float* q_gain,
                         const float* k_gain, float eps, uint32_t flags, hipStream_t stream);

/*
 * vdit_rope_qkv -- vdit_rope_qk plus the values of the same tokens in the
 * same launch: a decode step's three input transforms at once.
 *
 * q and k are treated exactly as by vdit_rope_qk (same flags, same results
 * bit for bit).  The values are not rotated: every v row is copied to v_out
 * unchanged, or, with VDIT_ROPE_V_NORM, normalised as by vdit_rms_norm,
 * y = x / sqrt(mean_d(x_d^2) + eps) * v_gain (KV-norm: FlashDecoder Sec. 3.2
 * "Base Architecture" normalises keys and values inside attention; the same
 * bits as vdit_rms_norm).  A rolling-cache slot of a B = 1 cache is a valid
 * k_out and v_out, so one call fills a decode frame's two slots.
 *
 * v_in, v_out: [B, L, n_kv_heads, head_dim] of dtype, both set or both
 * NULL (then this is vdit_rope_qk); v_out may equal v_in (in place) and must
 * not overlap any other tensor of the call.  v_gain: [head_dim] float32 or
 * NULL (gain 1), 16-byte aligned.  The other arguments as for vdit_rope_qk.
 * One workgroup holds a token's rows: the head rows of the tensors given
 * (n_heads for q, n_kv_heads each for k and v) times head_dim must not
 * exceed 16384 (VDIT_ERR_UNSUPPORTED beyond; the same limit as
 * vdit_rope_qk's).  VDIT_ROPE_V_NORM passed to vdit_rope_qk is an error.
 */
vdit_status vdit_rope_qkv(const void* q_in, const void* k_in, const void* v_in, void* q_out, void* k_out,
                          void* v_out, int32_t B, int64_t L, int32_t n_heads, int32_t n_kv_heads,
                          int32_t head_dim, vdit_dtype dtype, const vdit_grid* grid, int64_t token0,
                          int64_t t_offset, const float* q_gain, const float* k_gain, const float* v_gain,
                          float eps, uint32_t flags, hipStream_t stream);

/*
 * vdit_rms_norm -- per-head RMSNorm without rotation, for the values of
 * KV-norm attention (FlashDecoder Sec. 3.2 "Base Architecture" normalises
 * keys and values inside attention; the keys take the norm in vdit_rope_qk,
 * before their rotation, and the queries skip it with VDIT_ROPE_NO_Q_NORM).
 *
 * For every token and head: y = x / sqrt(mean_d(x_d^2) + eps) * gain.
 * x_in, x_out: [B, L, n_heads, head_dim] of dtype; x_out may equal x_in (in
 * place), partial overlap is not allowed.  A rolling-cache slot of a B = 1
 * cache is a valid x_out, so a decode step can normalise its values straight
 * into the cache.  gain: [head_dim] float32 or NULL (gain 1), 16-byte
 * aligned.  eps >= 0; head_dim in {64, 128}.  With B * L = 0 nothing is
 * done and x_in, x_out may be NULL.
 */
vdit_status vdit_rms_norm(const void* x_in, void* x_out, int32_t B, int64_t L, int32_t n_heads,
                          int32_t head_dim, vdit_dtype dtype, const float* gain, float eps,
                          hipStream_t stream);

typedef enum {
  VDIT_ATTN_FULL = 0,
  VDIT_ATTN_RING = 1,
  VDIT_ATTN_ROLLING = 2,
  VDIT_ATTN_CHUNK_HYBRID = 3
} vdit_attn_mode;

/*
 * Arguments of vdit_attn_fwd (host struct, read during the call only).
 * Query head h reads key/value head h / (n_heads / n_kv_heads) (grouped-query
 * attention, FlashDecoder Sec. 3.2).  Scores are s_ij = scale * q_i . k_j
 * with scale <= 0 meaning 1/sqrt(head_dim).
 *
 * VDIT_ATTN_FULL: O = softmax(S) V over all Lkv keys, no mask.
 *   q, o [B, Lq, n_heads, D]; k, v [B, Lkv, n_kv_heads, D]; lse optional.
 *
 * VDIT_ATTN_RING: one device's share of ring attention (ReGenVC:
 *   End-to-End Real-Time Generative Video Coding at Ultra-Low Bitrate,
 *   unified sequence parallelism paragraph): the key/value sequence is
 *   given as n_kv_chunks chunks whose partials are combined with the
 *   log-sum-exp merge of vdit_lse_merge.  k_chunks[c], v_chunks[c] (host
 *   arrays of device pointers) are [B, chunk_len[c], n_kv_heads, D];
 *   chunk_len (host) must sum to Lkv; k and v are unused.  Equal to FULL
 *   over the concatenated chunks up to rounding order.  Two forms:
 *   - fold (the ring's own order): one launch per chunk, in chunk order,
 *     each folding its partial into a float32 running partial in
 *     `workspace` (the merge is fused into the attention epilogue); the
 *     last chunk writes o and lse.  Chunk c is read only by launch c.  Taken
 *     for float32, for more than 8 chunks, with the VDIT_ATTN_RING_FOLD flag
 *     (vdit_attn_workspace_bytes then counts no one-launch partials), or
 *     when the workspace holds only the running partial.
 *   - one launch (bf16, 2..8 chunks, the default when the workspace holds a
 *     float32 partial per chunk): every chunk is attended to in one launch,
 *     whose workgroups cover (chunk, query tile, head), and the partials are
 *     merged afterwards; every chunk must be in place when the launch runs.
 *
 * VDIT_ATTN_ROLLING: frame-by-frame decode with a rolling KV cache of
 *   n_slots frames (FlashDecoder Sec. 3.3).  k_cache, v_cache are
 *   [B, n_slots, Lq, n_kv_heads, D]; frame f's keys/values live in slot
 *   f mod n_slots.  If k and v are non-NULL they hold frame `frame`'s
 *   [B, Lq, n_kv_heads, D] keys/values and are first copied into that slot;
 *   if both are NULL the slot was already filled (for example by passing it
 *   as k_out of vdit_rope_qk when B = 1).  q (frame `frame`'s queries,
 *   Lq = tokens per frame) then attends to the min(frame + 1, n_slots) most
 *   recent frames with no mask; Lkv is ignored.  Rotating each frame once at
 *   insertion with its absolute t gives the same scores as window-relative
 *   positions, because rotary scores depend only on position differences.
 *
 * VDIT_ATTN_CHUNK_HYBRID: softmax attention inside chunks of chunk_tokens
 *   tokens plus causal linear attention across chunks with running state
 *   (MobileWan: Closing the Quality Gap for Mobile Video Diffusion, review
 *   of Sec. 3.2).  Token i of chunk c gets
 *     (sum_{j in W_c} e^{s_ij} v_j + phi(q_i)^T S_c) / (sum_{j in W_c} e^{s_ij} + phi(q_i)^T z_c)
 *   with phi(x) = elu(x) + 1 on the (already normalised and rotated) q and k.
 *   The softmax window W_c is the chunk's own tokens plus the overlap_tokens
 *   keys before them (the review's appendix ledger: chunks of T_c temporal
 *   slices overlapping by T_o slices for the softmax attention; 0 = no
 *   overlap), and S_c = s_in + sum_{j before W_c} phi(k_j) v_j^T,
 *   z_c = z_in + sum_{j before W_c} phi(k_j): every key enters once.
 *   k, v hold Lkv = ctx_tokens + Lq tokens: the first ctx_tokens
 *   (0 <= ctx_tokens <= overlap_tokens) are keys/values from before the
 *   first query, which a streaming caller carries over from its previous
 *   call.  state_s [B, n_kv_heads, D, D] and state_z [B, n_kv_heads, D]
 *   (float32) hold the incoming state (zero for a new sequence; with the
 *   flag VDIT_ATTN_STATE_ZERO the incoming state is taken as zero and the
 *   two arrays are only written) and receive it with every key of the
 *   call folded in except the last overlap_tokens
 *   (the next call's context), so calling once per chunk equals one call
 *   over the whole sequence.  Needs `workspace` of
 *   vdit_attn_workspace_bytes().
 *   phi_coef (host array read during the call, or NULL): the review's ledger
 *   gives phi_q, phi_k as learnable polynomials of degree 3 (Appendix A.3.1
 *   as quoted there) without coefficients.  With phi_coef = (a0, a1, a2, a3,
 *   b0, b1, b2, b3), phi_q(x) = a0 + a1 x + a2 x^2 + a3 x^3 on each element
 *   of q and phi_k(x) = b0 + b1 x + b2 x^2 + b3 x^3 on each element of k
 *   replace elu + 1 (the state then sums phi_k(k) v^T and phi_k(k)).  The
 *   normaliser phi_q(q)^T z_c must be positive for the linear term to take
 *   part: choose coefficients that keep both maps positive on the values
 *   fed (after an RMSNorm with gain 1 every element lies in
 *   [-sqrt(D), sqrt(D)]); a row whose normaliser is not positive gets the
 *   softmax partial alone.  Coefficients must be finite.  NULL in the other
 *   modes.
 *
 * lse: [B, n_heads, Lq] float32 or NULL.  The ranges a call writes (o,
 * lse, the workspace_bytes bytes at workspace, the rolling caches, the
 * hybrid state) must not overlap one another or any other tensor of the
 * call (tensors that are only read may overlap); the one exception is a
 * ROLLING call with B = 1 passing the cache slot itself as k, v.  All of
 * this is checked before anything is enqueued.  workspace: 16-byte aligned
 * device scratch of at least vdit_attn_workspace_bytes(args) bytes (may be
 * NULL when that is 0); its contents need no initialisation and are
 * clobbered.  RING (with more than one chunk) and CHUNK_HYBRID require it.
 * For FULL and ROLLING it is optional: bf16 calls with too few queries to
 * occupy the device (fewer than two 128-query blocks per compute unit)
 * split the keys into up to 8 ranges, and calls of several rounds of such
 * blocks whose last round would be at most half full (more than three
 * blocks per compute unit, at least 8192 keys) into two; the ranges'
 * float32 partials live in the workspace and are merged with the
 * log-sum-exp combination of vdit_lse_merge.  Without a large enough
 * workspace these calls run unsplit (same result up to rounding order).
 *
 * key_norm_max: 0, or a bound the caller guarantees on the Euclidean norm of
 * every key of the call.  bf16 calls bound each query's scores by
 * |q_i| max_j |k_j| (Cauchy-Schwarz) and, where that bound keeps every
 * exponent within 32 binary orders of magnitude, run the softmax of those
 * queries without a running maximum; max_j |k_j| otherwise comes from one
 * pass over the keys (into the workspace, when it is large enough).  A
 * positive key_norm_max replaces that pass: for keys RMS-normalised with
 * gain 1 by vdit_rope_qk, sqrt(head_dim) * (1 + 2^-7) covers the bf16
 * rounding.  A value above the true maximum can only send more queries to
 * the running-maximum path.  One below it costs time, not correctness: a
 * true bound keeps every row sum of the bounded path within [2^-64, 2^64],
 * and a wavefront whose row sums leave that range (overflow, or its largest
 * terms lost to underflow) is detected when its workgroup has seen all its
 * keys; the workgroup then runs its keys once more on the running maximum.
 * Negative or non-finite: VDIT_ERR_INVALID_ARG.  Ignored by float32 calls.
 */
typedef struct {
  int32_t mode;  /* vdit_attn_mode */
  int32_t dtype; /* vdit_dtype of q, k, v, o, caches */
  int32_t B, n_heads, n_kv_heads, head_dim;
  int64_t Lq, Lkv;
  float scale;
  int32_t n_kv_chunks; /* RING */
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* const* k_chunks; /* RING (host array) */
  const void* const* v_chunks; /* RING (host array) */
  const int64_t* chunk_len;    /* RING (host array) */
  void* k_cache;               /* ROLLING */
  void* v_cache;               /* ROLLING */
  int64_t frame;               /* ROLLING */
  int32_t n_slots;             /* ROLLING */
  uint32_t flags;              /* VDIT_ATTN_* flags below (0: none) */
  int64_t chunk_tokens;        /* CHUNK_HYBRID */
  float* state_s;              /* CHUNK_HYBRID */
  float* state_z;              /* CHUNK_HYBRID */
  void* workspace;
  size_t workspace_bytes;
  int64_t overlap_tokens;      /* CHUNK_HYBRID (0 in the other modes) */
  int64_t ctx_tokens;          /* CHUNK_HYBRID (0 in the other modes) */
  float key_norm_max;          /* 0 = computed (see above) */
  int32_t reserved1;
  const float* phi_coef;       /* CHUNK_HYBRID (host, 8 floats) or NULL = elu + 1 */
} vdit_attn_args;

/* vdit_attn_args.flags */
#define VDIT_ATTN_RING_FOLD 1u /* RING: fold the chunks one launch at a time, in
                                  order, even where one launch could take them all */
#define VDIT_ATTN_STATE_ZERO 2u /* CHUNK_HYBRID: the incoming state is zero (the
                                   first call of a sequence): state_s and state_z
                                   are written, never read */

/* Bytes of device workspace vdit_attn_fwd needs (RING, CHUNK_HYBRID) or can
 * use (FULL, ROLLING: the key split) for these arguments on the current
 * device (0 if none).  Returns (size_t)-1 for arguments that fail
 * validation. */
size_t vdit_attn_workspace_bytes(const vdit_attn_args* args /* host */);

/* Enqueue one attention call (see vdit_attn_args).  head_dim in {64, 128}. */
vdit_status vdit_attn_fwd(const vdit_attn_args* args /* host */, hipStream_t stream);

/*
 * vdit_attn_fwd_noalloc -- vdit_attn_fwd for callers that cannot allocate
 * device memory (code under graph capture, serving loops, harnesses that
 * forbid allocation): the workspace is the library's own device scratch, a
 * static array of 64 MiB per device (held until the process ends), instead
 * of a caller's buffer.  args->workspace must be NULL and workspace_bytes 0
 * (else VDIT_ERR_INVALID_ARG); a call whose required workspace (RING with
 * several chunks, CHUNK_HYBRID: the part vdit_attn_workspace_bytes reports
 * beyond the optional key-norm and key-split areas) exceeds 64 MiB fails
 * with VDIT_ERR_UNSUPPORTED before anything is enqueued.  The optional areas
 * are used when they fit.  Results are those of vdit_attn_fwd with a
 * workspace of that size.  Allocates nothing: the scratch's device address
 * is looked up on the first call on each device.  All calls on one device
 * share the scratch, so calls that overlap in time on one device (several
 * streams or threads) race; serialise them.
 */
vdit_status vdit_attn_fwd_noalloc(const vdit_attn_args* args /* host */, hipStream_t stream);

/*
 * vdit_lse_merge -- combine two attention partials over disjoint key sets:
 *   L = ln(e^{L_a} + e^{L_b}),  O = e^{L_a - L} O_a + e^{L_b - L} O_b,
 * the online-softmax combination of ring attention (ReGenVC, USP
 * paragraph).  A partial with L = -inf has weight 0.  o_a, o_b: [B, L,
 * n_heads, head_dim] of in_dtype; lse_a, lse_b: [B, n_heads, L] float32;
 * o_out of out_dtype; lse_out may be NULL.  o_out may equal o_a (or o_b)
 * when in_dtype == out_dtype, and lse_out may equal lse_a (or lse_b).
 * head_dim in {64, 128}.
 */
vdit_status vdit_lse_merge(const void* o_a, const float* lse_a, const void* o_b,
                           const float* lse_b, void* o_out, float* lse_out,
                           vdit_dtype in_dtype, vdit_dtype out_dtype, int32_t B, int64_t L,
                           int32_t n_heads, int32_t head_dim, hipStream_t stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* vdit_last_error(void);

/* VDIT_ABI_VERSION of the loaded library. */
int32_t vdit_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VDIT_H */
