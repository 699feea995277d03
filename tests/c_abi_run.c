/* Plain C11 caller that runs the library's kernels through the C ABI: it
 * allocates device buffers with the HIP runtime, fills fp32 inputs from a
 * seeded generator, calls ln_fwd, bias_dropout_residual_ln_fwd (with the
 * mask written out), ln_bwd_dx with its partials and ln_bwd_dgamma_dbeta on
 * the ready partials, and writes inputs and outputs to a binary file for the
 * test to check against the float64 oracle.
 * Usage: c_abi_run ROWS COLS SEED OUT_PATH.  Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mbrow_ln.h"

static uint64_t st;
static float uniform(void) {   /* splitmix64 -> [0, 1) */
    st += 0x9E3779B97F4A7C15ull;
    uint64_t z = st;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (float)((double)(z >> 40) / 16777216.0);
}

#define CHECK_HIP(e)                                                         \
    do {                                                                     \
        hipError_t err_ = (e);                                               \
        if (err_ != hipSuccess) {                                            \
            fprintf(stderr, "HIP error %d at line %d\n", (int)err_, __LINE__); \
            return 2;                                                        \
        }                                                                    \
    } while (0)
#define CHECK_LN(e)                                                          \
    do {                                                                     \
        ln_status_t s_ = (e);                                                \
        if (s_ != LN_OK) {                                                   \
            fprintf(stderr, "%s at line %d\n", ln_status_string(s_), __LINE__); \
            return 3;                                                        \
        }                                                                    \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 5) {
        fprintf(stderr, "usage: c_abi_run ROWS COLS SEED OUT_PATH\n");
        return 1;
    }
    const int64_t rows = atoll(argv[1]), cols = atoll(argv[2]);
    st = strtoull(argv[3], NULL, 10);
    if (rows <= 0 || cols <= 0 || rows * cols > (1 << 24)) return 1;
    const size_t n = (size_t)(rows * cols), nb = n * sizeof(float), cb = (size_t)cols * sizeof(float);
    const float eps = 1e-5f, p = 0.1f;
    const uint64_t seed = 12345;

    /* host inputs: x, residual, dy ~ U(-2, 2); gamma ~ U(0.5, 1.5); beta, bias ~ U(-0.1, 0.1) */
    float* h = (float*)malloc(nb * 3 + cb * 3);
    float *hx = h, *hr = h + n, *hdy = h + 2 * n, *hg = h + 3 * n, *hb = hg + cols, *hbias = hb + cols;
    for (size_t i = 0; i < 3 * n; ++i) h[i] = 4.0f * uniform() - 2.0f;
    for (int64_t j = 0; j < cols; ++j) {
        hg[j] = 0.5f + uniform();
        hb[j] = 0.2f * uniform() - 0.1f;
        hbias[j] = 0.2f * uniform() - 0.1f;
    }

    float *x, *r, *dy, *g, *b, *bias, *y, *z, *y2, *dx, *mean, *rstd, *mean2, *rstd2, *dg, *db, *ws;
    uint8_t* mask;
    const size_t wsb = ln_bwd_workspace_bytes(rows, cols);
    CHECK_HIP(hipMalloc((void**)&x, nb));
    CHECK_HIP(hipMalloc((void**)&r, nb));
    CHECK_HIP(hipMalloc((void**)&dy, nb));
    CHECK_HIP(hipMalloc((void**)&g, cb));
    CHECK_HIP(hipMalloc((void**)&b, cb));
    CHECK_HIP(hipMalloc((void**)&bias, cb));
    CHECK_HIP(hipMalloc((void**)&y, nb));
    CHECK_HIP(hipMalloc((void**)&z, nb));
    CHECK_HIP(hipMalloc((void**)&y2, nb));
    CHECK_HIP(hipMalloc((void**)&dx, nb));
    CHECK_HIP(hipMalloc((void**)&mean, (size_t)rows * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&rstd, (size_t)rows * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&mean2, (size_t)rows * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&rstd2, (size_t)rows * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&dg, cb));
    CHECK_HIP(hipMalloc((void**)&db, cb));
    CHECK_HIP(hipMalloc((void**)&ws, wsb));
    CHECK_HIP(hipMalloc((void**)&mask, n));
    CHECK_HIP(hipMemcpy(x, hx, nb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(r, hr, nb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dy, hdy, nb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(g, hg, cb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(b, hb, cb, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(bias, hbias, cb, hipMemcpyHostToDevice));

    CHECK_LN(ln_fwd(x, g, b, y, mean, rstd, rows, cols, eps, LN_F32, NULL));
    CHECK_LN(bias_dropout_residual_ln_fwd(x, bias, r, g, b, z, y2, mean2, rstd2, mask, rows, cols,
                                          eps, p, seed, LN_F32, NULL));
    CHECK_LN(ln_bwd_dx(dy, x, g, mean, rstd, dx, ws, wsb, rows, cols, LN_F32, NULL));
    CHECK_LN(ln_bwd_dgamma_dbeta(NULL, NULL, NULL, NULL, dg, db, ws, wsb, 1, rows, cols, LN_F32,
                                 NULL));
    CHECK_HIP(hipStreamSynchronize(NULL));

    /* file: inputs x, residual, dy, gamma, beta, bias; outputs y, mean, rstd,
     * z, y2, mean2, rstd2, dx, dgamma, dbeta (float32), then the mask (u8) */
    FILE* f = fopen(argv[4], "wb");
    if (!f) return 4;
    fwrite(h, 1, nb * 3 + cb * 3, f);
    float* buf = (float*)malloc(nb);
    uint8_t* mb = (uint8_t*)malloc(n);
    const float* dev[] = {y, mean, rstd, z, y2, mean2, rstd2, dx, dg, db};
    const size_t len[] = {nb, rows * sizeof(float), rows * sizeof(float), nb, nb,
                          rows * sizeof(float), rows * sizeof(float), nb, cb, cb};
    for (int i = 0; i < 10; ++i) {
        CHECK_HIP(hipMemcpy(buf, dev[i], len[i], hipMemcpyDeviceToHost));
        fwrite(buf, 1, len[i], f);
    }
    CHECK_HIP(hipMemcpy(mb, mask, n, hipMemcpyDeviceToHost));
    fwrite(mb, 1, n, f);
    fclose(f);

    hipFree(x); hipFree(r); hipFree(dy); hipFree(g); hipFree(b); hipFree(bias); hipFree(y);
    hipFree(z); hipFree(y2); hipFree(dx); hipFree(mean); hipFree(rstd); hipFree(mean2);
    hipFree(rstd2); hipFree(dg); hipFree(db); hipFree(ws); hipFree(mask);
    free(h); free(buf); free(mb);
    printf("c_abi_run: ok\n");
    return 0;
}
