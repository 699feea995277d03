/* Plain C11 user of the C ABI: compiles against include/mbrow_ln.h with a C
 * compiler, links against the library, and calls every entry point with
 * arguments the library rejects on the host (so nothing reaches a GPU).
 * Prints one line per check and exits nonzero on the first mismatch. */
#include <stdint.h>
#include <stdio.h>

#include "mbrow_ln.h"

static int fails = 0;

static void expect(const char* what, ln_status_t got, ln_status_t want) {
    printf("%-32s %d %s\n", what, (int)got, ln_status_string(got));
    if (got != want) {
        printf("  expected %d\n", (int)want);
        ++fails;
    }
}

int main(void) {
    void* a = (void*)(uintptr_t)0x10000000u;   /* non-NULL, never dereferenced */
    float* f = (float*)(uintptr_t)0x20000000u;
    const int64_t* lab = (const int64_t*)(uintptr_t)0x30000000u;
    hipStream_t s = NULL;

    expect("ln_fwd null", ln_fwd(NULL, a, a, a, NULL, NULL, 4, 8, 1e-5f, LN_BF16, s), LN_ERR_NULL);
    expect("bias_dropout_residual_ln_fwd p",
           bias_dropout_residual_ln_fwd(a, a, a, a, a, a, a, NULL, NULL, NULL, 4, 8, 1e-5f, 1.5f,
                                        0, LN_BF16, s),
           LN_ERR_PARAM);
    expect("ln_bwd_dx shape", ln_bwd_dx(a, a, a, f, f, a, NULL, 0, -1, 8, LN_F32, s),
           LN_ERR_SHAPE);
    expect("ln_bwd_dgamma_dbeta workspace",
           ln_bwd_dgamma_dbeta(a, a, f, f, f, f, f, 4, 0, 4, 8, LN_F16, s), LN_ERR_WORKSPACE);
    expect("bias_dropout_residual_ln_bwd dtype",
           bias_dropout_residual_ln_bwd(a, NULL, a, a, f, f, a, a, f, f, f, f, 1 << 20, 4, 8,
                                        0.1f, 0, (ln_dtype_t)9, s),
           LN_ERR_DTYPE);
    expect("attn_softmax_fwd causal",
           attn_softmax_fwd(a, NULL, 1, a, NULL, 4, 8, 1.0f, 2, 0.0f, 0, LN_F16, s), LN_ERR_PARAM);
    expect("attn_softmax_bwd null",
           attn_softmax_bwd(NULL, a, a, 4, 8, 1.0f, 0, 0.0f, 0, LN_F16, s), LN_ERR_NULL);
    expect("add_rmsnorm_fwd eps",
           add_rmsnorm_fwd(a, NULL, a, NULL, a, NULL, 4, 8, -1.0f, LN_BF16, s), LN_ERR_PARAM);
    expect("add_rmsnorm_bwd null",
           add_rmsnorm_bwd(a, NULL, a, a, f, a, NULL, f, 1 << 20, 4, 8, LN_BF16, s), LN_ERR_NULL);
    expect("cross_entropy_fwd_bwd ld",
           cross_entropy_fwd_bwd(a, lab, f, NULL, 4, 8, 7, 0.0f, 1.0f, LN_BF16, s), LN_ERR_SHAPE);
    expect("empty call", ln_fwd(a, a, a, a, NULL, NULL, 0, 8, 1e-5f, LN_BF16, s), LN_OK);
    expect("hbm_copy size", hbm_copy(a, f, 20, s), LN_ERR_PARAM);
    expect("hbm_copy null", hbm_copy(NULL, f, 16, s), LN_ERR_NULL);
    expect("hbm_copy empty", hbm_copy(a, f, 0, s), LN_OK);

    if (ln_bwd_workspace_bytes(8192, 1280) != (size_t)256 * 2 * 1280 * 4) ++fails;
    if (bias_dropout_residual_ln_bwd_workspace_bytes(8192, 1280) != (size_t)256 * 3 * 1280 * 4)
        ++fails;
    if (add_rmsnorm_bwd_workspace_bytes(8192, 1280) != (size_t)256 * 1280 * 4) ++fails;
    printf("%s\n", fails ? "FAILED" : "OK");
    return fails ? 1 : 0;
}
