/* A plain C99 caller of libusp.so: the header compiles as C, and the
 * library's synchronous validation answers without a GPU (no kernel is
 * launched by any call below).  Exits 0 and prints "abi ok" on success. */
#include <stdio.h>
#include <string.h>

#include "usp.h"

static int failures = 0;

static void expect(int cond, const char *what) {
  if (!cond) {
    fprintf(stderr, "FAIL: %s (detail: %s)\n", what, usp_last_error_detail());
    ++failures;
  }
}

int main(void) {
  /* never dereferenced: validation rejects every call before a launch */
  void *a = (void *)0x10000, *b = (void *)0x20000;
  expect(usp_abi_version() == USP_ABI_VERSION, "library and header agree on the ABI version");
  expect(strcmp(usp_status_string(USP_ERR_INVALID_ARG), "USP_ERR_INVALID_ARG") == 0, "status string");

  /* zigzag: null input, then a sequence that 2 rd ud does not divide */
  expect(usp_zigzag_extract(NULL, b, USP_DTYPE_BF16, 1, 64, 2, 64, 4, 1, 0, 0, 0, NULL) == USP_ERR_INVALID_ARG,
         "zigzag_extract rejects a null input");
  expect(strlen(usp_last_error_detail()) > 0, "a rejected call leaves a message");
  expect(usp_zigzag_extract(a, b, USP_DTYPE_BF16, 1, 60, 2, 64, 4, 1, 0, 0, 0, NULL) == USP_ERR_INVALID_ARG,
         "zigzag_extract rejects S % (2 rd ud) != 0");

  /* batched copies: n out of range, and an output inside an input */
  {
    const void *xs[2] = {a, b};
    void *outs[2] = {(char *)a + 0x100000, (char *)a + 16};
    const int64_t heads[2] = {2, 2};
    expect(usp_zigzag_extract_n(0, xs, outs, heads, USP_DTYPE_BF16, 1, 64, 64, 4, 1, 0, 0, 0, NULL) ==
               USP_ERR_INVALID_ARG, "zigzag_extract_n rejects n = 0");
    expect(usp_zigzag_extract_n(2, xs, outs, heads, USP_DTYPE_BF16, 1, 64, 64, 4, 1, 0, 0, 0, NULL) ==
               USP_ERR_INVALID_ARG, "zigzag_extract_n rejects an output overlapping an input");
  }

  /* Ulysses layout: heads not divisible by the degree */
  expect(usp_ulysses_a2a_layout(a, b, USP_DTYPE_BF16, 1, 64, 3, 64, 2, 0, 0, NULL) == USP_ERR_INVALID_ARG,
         "ulysses_a2a_layout rejects hc % N != 0");

  /* attention: an unsupported head dim, then a rank out of range */
  {
    usp_attn_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 1;
    d.seq_len = 256;
    d.num_q_heads = 2;
    d.num_kv_heads = 2;
    d.head_dim = 96;
    d.dtype = USP_DTYPE_BF16;
    d.softmax_scale = 0.125f;
    d.causal = 1;
    d.cp = 4;
    /* (B, 2c, H, D) shares of 64 tokens; the KV blocks one share apart */
    d.q.s = d.k.s = d.v.s = d.o.s = 2 * 64;
    d.q.h = d.k.h = d.v.h = d.o.h = 64;
    d.q.b = d.k.b = d.v.b = d.o.b = 64 * 2 * 64;
    d.kv_block_stride = 64 * 2 * 64;
    expect(usp_attn_fwd(a, b, a, b, (float *)a, &d, 0, NULL) == USP_ERR_UNSUPPORTED, "attn_fwd rejects head_dim 96");
    expect(strstr(usp_last_error_detail(), "head_dim") != NULL, "the message names head_dim");
    d.head_dim = 64;
    expect(usp_attn_fwd_split_workspace(&d, 0) == 2 * 2 * 64 * (d.head_dim + 1) * 4,
           "split walk workspace: two partials of every row");
    expect(usp_attn_fwd_split_workspace(NULL, 0) == -1, "split walk workspace rejects a null descriptor");
    expect(usp_attn_fwd_split(a, b, a, b, (float *)a, &d, 0, NULL, 1 << 20, NULL) == USP_ERR_INVALID_ARG,
           "attn_fwd_split rejects a null workspace");
    expect(usp_attn_fwd(a, b, a, b, (float *)a, &d, 4, NULL) == USP_ERR_INVALID_ARG,
           "attn_fwd rejects ring_rank = cp");
    expect(strstr(usp_last_error_detail(), "ring_rank") != NULL, "the message names ring_rank");
  }

  if (failures) return 1;
  printf("abi ok\n");
  return 0;
}
