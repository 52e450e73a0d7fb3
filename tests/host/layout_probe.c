/* Prints the layout of the public structs of include/vdit.h as seen by a C
 * compiler, so the Python binding's ctypes mirror can be checked against it. */
#include <stddef.h>
#include <stdio.h>
#include "vdit.h"

int main(void) {
  printf("vdit_grid %zu\n", sizeof(vdit_grid));
  printf("vdit_attn_args %zu\n", sizeof(vdit_attn_args));
#define OFF(f) printf("%s %zu\n", #f, offsetof(vdit_attn_args, f))
  OFF(mode); OFF(dtype); OFF(B); OFF(n_heads); OFF(n_kv_heads); OFF(head_dim);
  OFF(Lq); OFF(Lkv); OFF(scale); OFF(n_kv_chunks); OFF(q); OFF(k); OFF(v); OFF(o); OFF(lse);
  OFF(k_chunks); OFF(v_chunks); OFF(chunk_len); OFF(k_cache); OFF(v_cache); OFF(frame);
  OFF(n_slots); OFF(flags); OFF(chunk_tokens); OFF(state_s); OFF(state_z); OFF(workspace);
  OFF(workspace_bytes); OFF(overlap_tokens); OFF(ctx_tokens); OFF(key_norm_max); OFF(reserved1); OFF(phi_coef);
  return 0;
}
