/* The C ABI used from plain C99 (test infrastructure): compiled with gcc
 * against include/fa16attn.h and linked with libfa16attn.so. It calls only
 * what needs no GPU: the version, the error strings, the workspace queries
 * and argument rejections, which the library reports before any HIP call.
 * Prints "OK" and exits 0 when every check holds; otherwise names the first
 * failing check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "fa16attn.h"

static int failures = 0;

static void check(int ok, const char* what)
{
    if (!ok && failures++ == 0) printf("FAIL %s\n", what);
}

int main(void)
{
    check(fa_abi_version() == FA16ATTN_ABI_VERSION, "abi version");
    for (int c = 0; c <= 6; ++c) check(fa_error_string(c) != NULL && strlen(fa_error_string(c)) > 0, "error string");
    check(fa_error_string(FA_ERR_HIP + 1) != NULL, "error string of a HIP code");

    /* the causal prefill of 8000 rows against 128000 keys at D256: two key segments per query tile */
    check(attn_fwd_prefix_causal_workspace(1, 6, 1, 256, 8000, 128000) == (size_t)2 * 6 * 8000 * (256 * 4 + 8),
          "causal workspace");
    check(attn_fwd_prefix_causal_workspace(1, 6, 1, 256, 100, 128000) == 0, "causal workspace of an invalid shape");
    size_t base = attn_fwd_paged_e4m3_workspace(1, 6, 1, 256, 8000, 256000);
    size_t partial = (base + 255) / 256 * 256;
    check(attn_fwd_paged_e4m3_bridged_workspace(1, 6, 1, 256, 8000, 256000, 0.0703418f) ==
              partial + (size_t)4 * 256000 * 256,
          "bridged workspace");
    check(attn_fwd_paged_e4m3_bridged_workspace(1, 6, 1, 256, 8000, 256000, 0.0625f) == base,
          "bridged workspace of a power-of-two scale");
    check(attn_fwd_paged_e4m3_decode_workspace(1, 6, 1, 256, 16, 256000) > 0, "decode workspace");
    check(vsa_block_select_workspace(1, 8, 36864, 128, 64) > 0, "selection workspace");

    /* rejections before any HIP call */
    fa_tensor none = {NULL, 0, 0, 0};
    check(attn_fwd_dense(none, none, none, none, NULL, 1, 1, 16, 16, 128, 0.088f, NULL) == FA_ERR_NULL,
          "dense with NULL tensors");
    check(vsa_topk_for_sparsity(36864, 64, 0.8) == 116, "keep ratio 0.2 of 576 blocks");
    check(kv_e4m3_paged_to_fp16(NULL, NULL, NULL, 1, 1, 32, 1, 1, 128, 32, 1.f, 1.f, NULL, NULL, NULL) == FA_ERR_NULL,
          "bridge with NULL pointers");

    if (failures) return 1;
    printf("OK\n");
    return 0;
}
