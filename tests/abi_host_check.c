/* Host paths of the C ABI, for the sanitized build of the library
 * (tests/test_sanitized_host.py builds this with address and
 * undefined-behaviour sanitizers and links it against
 * _build/sanitized/libbsattn.so). Runs without a GPU: every call either fails
 * host-side validation or reaches the device check, which reports that no
 * device is present. Fake device pointers are never dereferenced.
 *
 * Prints one "name status" line per call, then "last <message>" lines. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bsattn.h"

static void *const FAKE = (void *)(uintptr_t)(1ull << 40);

static attn_shape edge48k(void) {
  attn_shape s;
  memset(&s, 0, sizeof s);
  s.batch = 1; s.num_q_heads = 32; s.num_kv_heads = 8; s.head_dim = 128;
  s.block_q = 64; s.block_k = 64; s.q_len = 48384; s.q_valid = 48360;
  s.kv_prefix_len = 512; s.kv_prefix_valid = 512; s.kv_len = 48896; s.kv_suffix_valid = 48360;
  const int64_t qs[3] = {48384LL * 32 * 128, 32 * 128, 128};
  const int64_t ks[3] = {48896LL * 8 * 128, 8 * 128, 128};
  for (int i = 0; i < 3; ++i) {
    s.q_stride[i] = qs[i]; s.o_stride[i] = qs[i]; s.k_stride[i] = ks[i]; s.v_stride[i] = ks[i];
  }
  return s;
}

#define SHOW(name, expr) printf("%s %d\n", name, (int)(expr))

int main(void) {
  attn_shape s = edge48k();
  const size_t ws = attn_select_workspace_size(&s);
  int32_t *I = (int32_t *)FAKE;
  SHOW("keep", attn_keep_blocks(764, 8, 75));
  SHOW("keep_bad", attn_keep_blocks(-1, 0, 75));
  SHOW("support", attn_query_support(&s));
  SHOW("support_null", attn_query_support(NULL));
  SHOW("ws_positive", ws > 0);

  attn_shape bad = s; bad.num_q_heads = 30;            /* not a multiple of Hkv */
  SHOW("support_group", attn_query_support(&bad));
  bad = s; bad.head_dim = 96;
  SHOW("support_hd", attn_query_support(&bad));
  bad = s; bad.q_len = 48383;
  SHOW("support_qlen", attn_query_support(&bad));
  bad = s; bad.k_stride[1] = 1030;                    /* not a multiple of 8 */
  SHOW("support_stride", attn_query_support(&bad));
  bad = s; bad.softmax_scale = -1.0f;                 /* <= 0: the default scale */
  SHOW("support_scale_default", attn_query_support(&bad));
  bad = s; bad.softmax_scale = __builtin_nanf("");
  SHOW("support_scale_nan", attn_query_support(&bad));
  SHOW("ws_bad", attn_select_workspace_size(&bad) == 0);

  /* selector: keep out of range, stride below keep, workspace, pointers */
  SHOW("sel_keep", attn_select_blocks(&s, FAKE, FAKE, 7, I, I, 191, FAKE, ws, NULL));
  SHOW("sel_stride", attn_select_blocks(&s, FAKE, FAKE, 191, I, I, 190, FAKE, ws, NULL));
  SHOW("sel_ws", attn_select_blocks(&s, FAKE, FAKE, 191, I, I, 191, FAKE, ws - 1, NULL));
  SHOW("sel_null", attn_select_blocks(&s, NULL, FAKE, 191, I, I, 191, FAKE, ws, NULL));
  SHOW("sel_device", attn_select_blocks(&s, FAKE, FAKE, 191, I, I, 191, FAKE, ws, NULL));
  SHOW("noalloc_device", attn_select_blocks_noalloc(&s, FAKE, FAKE, 191, I, I, 191, NULL));

  /* attention: null lists, stride, misaligned output, then the device check */
  SHOW("bs_null", attn_block_sparse_fwd(&s, FAKE, FAKE, FAKE, NULL, I, 191, FAKE, NULL, NULL));
  SHOW("bs_stride", attn_block_sparse_fwd(&s, FAKE, FAKE, FAKE, I, I, 0, FAKE, NULL, NULL));
  SHOW("bs_align", attn_block_sparse_fwd(&s, FAKE, FAKE, FAKE, I, I, 191,
                                         (char *)FAKE + 2, NULL, NULL));
  SHOW("bs_device", attn_block_sparse_fwd(&s, FAKE, FAKE, FAKE, I, I, 191, FAKE, NULL, NULL));
  SHOW("dense_device", attn_dense_fwd(&s, FAKE, FAKE, FAKE, FAKE, NULL, NULL));
  SHOW("causal_device", attn_dense_causal_fwd(&s, FAKE, FAKE, FAKE, FAKE, NULL, NULL));
  SHOW("self_test", attn_self_test());

  /* strategy: the pages' mixed recipe (10 dense steps, layers 8-35 sparse) */
  attn_strategy st;
  st.num_layers = 36; st.dense_steps = 10; st.sparsity_pct = 75;
  st.sparse_layers = 0;
  for (int l = 8; l < 36; ++l) st.sparse_layers |= 1ull << l;
  SHOW("strat_dense_step", attn_strategy_is_sparse(&st, 3, 20));
  SHOW("strat_sparse", attn_strategy_is_sparse(&st, 10, 8));
  SHOW("strat_dense_layer", attn_strategy_is_sparse(&st, 10, 7));
  SHOW("strat_bad_layer", attn_strategy_is_sparse(&st, 10, 36));
  SHOW("strat_null", attn_strategy_is_sparse(NULL, 0, 0));
  const size_t sws = attn_strategy_workspace_size(&s, &st);
  SHOW("strat_ws_positive", sws > ws);
  SHOW("strat_ws_small", attn_strategy_fwd(&s, &st, 12, 9, FAKE, FAKE, FAKE, FAKE, NULL, FAKE,
                                           sws - 1, NULL));
  SHOW("strat_device", attn_strategy_fwd(&s, &st, 12, 9, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, sws,
                                         NULL));
  printf("last %s\n", attn_last_error());
  SHOW("support_again", attn_query_support(&s));
  printf("last [%s]\n", attn_last_error());
  printf("version %s\n", attn_version());
  return 0;
}
