/* Drives every function of the float64 oracle over small, ragged and edge
 * shapes (one column, one row, a fully masked causal row, ignored and
 * invalid labels, p = 0) in a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer, so that an out-of-bounds access, a use of
 * uninitialised heap memory through ASan's poisoning, a signed overflow or a
 * misaligned access in the oracle stops the program.  Test infrastructure
 * only: it links the oracle and nothing of the library. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ln_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double draw(void) {   /* splitmix64 -> [-2, 2) */
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (4.0 / 9007199254740992.0) - 2.0;
}
static double* vec(int64_t n) {
    double* v = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) v[i] = draw();
    return v;
}

static int shape(int64_t rows, int64_t m) {
    const int64_t n = rows * m;
    double *x = vec(n), *dy = vec(n), *res = vec(n), *y = vec(n), *dx = vec(n), *z = vec(n);
    double *g = vec(m), *b = vec(m), *bias = vec(m), *mask = vec(n);
    double *mean = vec(rows), *rstd = vec(rows), *var = vec(rows), *var2 = vec(rows);
    double *dg = vec(m), *db = vec(m), *sg = vec(m), *sb = vec(m), *loss = vec(rows);
    uint8_t* keep = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
    int64_t* lab = (int64_t*)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(int64_t));
    for (int64_t r = 0; r < rows; ++r) lab[r] = r % 3 == 1 ? -1 : (r % 5 == 4 ? m : r % m);

    orc_round_array(x, y, n, ORC_BF16);
    orc_round_array(x, y, n, ORC_F16);
    orc_ln_fwd(x, g, b, rows, m, 1e-5, y, mean, rstd);
    orc_ln_fwd(x, g, b, rows, m, 1e-5, NULL, NULL, NULL);
    orc_row_stats_welford(x, rows, m, mean, var);
    orc_var_naive_f32(x, rows, m, var);
    orc_var_chan_f32(x, rows, m, 4, var2);
    for (int i = 0; i < 3; ++i) {
        const float p = i == 0 ? 0.0f : (i == 1 ? 0.1f : 0.9f);
        orc_dropout_keep(0x0123456789ABCDEFull + (uint64_t)i, p, rows, m, keep);
        orc_dropout_keep_rows(7, p, 5, rows, m, keep);
        orc_bias_dropout_residual(x, bias, res, keep, p, rows, m, z);
        orc_dropout_residual_bwd(dy, keep, p, rows, m, dx, db, sb);
        orc_dropout_residual_bwd(dy, keep, p, rows, m, dx, db, NULL);
        orc_attn_softmax_bwd(dy, y, keep, p, rows, m, 0.5, dx);
    }
    orc_ln_fwd(x, g, b, rows, m, 1e-5, y, mean, rstd);
    orc_ln_bwd_dx_hw4(dy, x, g, mean, rstd, rows, m, dx);
    orc_ln_bwd_dx_scale(dy, x, g, mean, rstd, rows, m, z);
    orc_ln_bwd_dx_slides(dy, x, g, mean, rstd, rows, m, dx);
    orc_ln_bwd_params(dy, x, mean, rstd, rows, m, dg, db, sg, sb);
    orc_ln_bwd_params(dy, x, mean, rstd, rows, m, dg, db, NULL, NULL);
    orc_rmsnorm_fwd(x, g, rows, m, 1e-6, y, rstd);
    orc_rmsnorm_bwd(dy, x, g, rstd, rows, m, dx, dg, sg);
    orc_rmsnorm_bwd(dy, x, g, rstd, rows, m, dx, dg, NULL);
    orc_attn_softmax_fwd(x, NULL, 1, rows, m, 0.5, 0, y);
    orc_attn_softmax_fwd(x, mask, 1, rows, m, 0.5, 1, y);
    if (rows > 1) orc_attn_softmax_fwd(x, mask, rows, rows, m, 0.5, 0, y);
    orc_attn_softmax_bwd(dy, y, NULL, 0.0f, rows, m, 0.5, dx);
    orc_cross_entropy(x, lab, rows, m, 0.1, 1.0, loss, dx);
    orc_cross_entropy(x, lab, rows, m, 0.0, 0.5, loss, NULL);

    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    orc_philox4x32_10(ctr, key, out);
    const uint32_t thr = orc_dropout_threshold(0.1f);
    const double r = orc_round(1001.0, ORC_BF16) + orc_round(INFINITY, ORC_F16) +
                     orc_round(70000.0, ORC_F16);
    int bad = !(thr == 6554u) || !(r == INFINITY);

    free(x); free(dy); free(res); free(y); free(dx); free(z); free(g); free(b); free(bias);
    free(mask); free(mean); free(rstd); free(var); free(var2); free(dg); free(db); free(sg);
    free(sb); free(loss); free(keep); free(lab);
    return bad;
}

int main(void) {
    static const int64_t shapes[][2] = {{1, 1}, {1, 7}, {3, 1}, {5, 8}, {7, 33}, {16, 1000},
                                        {2, 4097}, {33, 64}};
    int bad = 0;
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        bad |= shape(shapes[i][0], shapes[i][1]);
    if (bad) {
        fprintf(stderr, "oracle_sanitize: unexpected values\n");
        return 1;
    }
    printf("oracle_sanitize: ok\n");
    return 0;
}
