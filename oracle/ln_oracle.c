/*
 * ln_oracle.c -- float64 CPU oracle for fused LayerNorm (test infrastructure).
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use this
 * file.  It is deliberately plain: one row at a time, one element at a time,
 * in the order the definitions are written, with no blocking, vectorisation
 * or fusion.  Sources are listed in ln_oracle.h.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared ln_oracle.c -lm
 * (-ffp-contract=off keeps every product and sum rounded as written).
 */
#include "ln_oracle.h"

#include <math.h>
#include <stddef.h>

/* ------------------------------------------------------------------------ */
/* Rounding to a storage format ([FP] §7.1-7.3, exercise 6).                 */
/* ------------------------------------------------------------------------ */

double orc_round(double v, int fmt) {
    int p, emin, emax; /* significant bits, smallest / largest normal exponent */
    switch (fmt) {
    case ORC_F32:  p = 24; emin = -126; emax = 127; break;
    case ORC_F16:  p = 11; emin = -14;  emax = 15;  break;
    case ORC_BF16: p = 8;  emin = -126; emax = 127; break;
    default: return NAN;
    }
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    int k;
    frexp(v, &k);              /* |v| = f * 2^k with f in [0.5, 1)       */
    int e = k - 1;             /* exponent with the significand in [1, 2) */
    if (e < emin) e = emin;    /* subnormal range keeps the fixed quantum */
    int qexp = e - (p - 1);    /* the spacing of the format near v is 2^qexp */
    double r = nearbyint(ldexp(v, -qexp)); /* round to nearest, ties to even */
    double out = ldexp(r, qexp);
    double maxfinite = ldexp(ldexp(1.0, p) - 1.0, emax - (p - 1));
    if (fabs(out) > maxfinite) return copysign(INFINITY, v);
    return out;
}

void orc_round_array(const double* in, double* out, int64_t n, int fmt) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_round(in[i], fmt);
}

/* ------------------------------------------------------------------------ */
/* Forward ([L11] §2.1, [L10] §4.2).                                         */
/* ------------------------------------------------------------------------ */

void orc_ln_fwd(const double* x, const double* gamma, const double* beta,
                int64_t rows, int64_t m, double eps,
                double* y, double* mean, double* rstd) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * m;
        double s = 0.0;
        for (int64_t j = 0; j < m; ++j) s += xr[j];
        double mu = s / (double)m;
        double ss = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double d = xr[j] - mu;
            ss += d * d;
        }
        double var = ss / (double)m;
        double rs = 1.0 / sqrt(var + eps);
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
        if (y) {
            for (int64_t j = 0; j < m; ++j) {
                double xhat = (xr[j] - mu) * rs;
                y[r * m + j] = gamma[j] * xhat + beta[j];
            }
        }
    }
}

/* One Welford pass over x[lo, hi): count, mean, sum of squared deviations. */
static void welford_range(const double* x, int64_t lo, int64_t hi,
                          double* n_out, double* mean_out, double* m2_out) {
    double n = 0.0, mu = 0.0, m2 = 0.0;
    for (int64_t j = lo; j < hi; ++j) {
        n += 1.0;
        double d = x[j] - mu;
        mu += d / n;
        m2 += d * (x[j] - mu);
    }
    *n_out = n; *mean_out = mu; *m2_out = m2;
}

void orc_row_stats_welford(const double* x, int64_t rows, int64_t m,
                           double* mean, double* var) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * m;
        double na, ma, m2a, nb, mb, m2b;
        welford_range(xr, 0, m / 2, &na, &ma, &m2a);
        welford_range(xr, m / 2, m, &nb, &mb, &m2b);
        double n = na + nb, mu, m2;
        if (na == 0.0) {
            mu = mb; m2 = m2b;
        } else {
            /* Chan merge, [L10] §4.2 */
            double delta = mb - ma;
            mu = ma + delta * nb / n;
            m2 = m2a + m2b + delta * delta * na * nb / n;
        }
        mean[r] = mu;
        var[r] = m2 / n;
    }
}

void orc_var_naive_f32(const double* x, int64_t rows, int64_t m, double* var) {
    for (int64_t r = 0; r < rows; ++r) {
        float s = 0.0f, ss = 0.0f;
        for (int64_t j = 0; j < m; ++j) {
            float v = (float)x[r * m + j];
            s += v;
            ss += v * v;
        }
        float mu = s / (float)m;
        float ex2 = ss / (float)m;
        var[r] = (double)(ex2 - mu * mu);
    }
}

void orc_var_chan_f32(const double* x, int64_t rows, int64_t m, int lanes,
                      double* var) {
    enum { MAXL = 1024 };
    float cnt[MAXL], mu[MAXL], m2[MAXL];
    if (lanes < 1 || lanes > MAXL || (lanes & (lanes - 1)) != 0) {
        for (int64_t r = 0; r < rows; ++r) var[r] = NAN;
        return;
    }
    for (int64_t r = 0; r < rows; ++r) {
        for (int l = 0; l < lanes; ++l) {
            float n = 0.0f, a = 0.0f, q = 0.0f;
            for (int64_t j = l; j < m; j += lanes) {
                float v = (float)x[r * m + j];
                n += 1.0f;
                float d = v - a;
                a += d / n;
                q += d * (v - a);
            }
            cnt[l] = n; mu[l] = a; m2[l] = q;
        }
        for (int stride = lanes / 2; stride >= 1; stride /= 2) {
            for (int l = 0; l < stride; ++l) {
                float na = cnt[l], nb = cnt[l + stride];
                if (nb == 0.0f) continue;
                if (na == 0.0f) {
                    cnt[l] = nb; mu[l] = mu[l + stride]; m2[l] = m2[l + stride];
                    continue;
                }
                float n = na + nb;
                float delta = mu[l + stride] - mu[l];
                mu[l] = mu[l] + delta * (nb / n);
                m2[l] = m2[l] + m2[l + stride] + delta * delta * (na * nb / n);
                cnt[l] = n;
            }
        }
        var[r] = (double)(m2[0] / cnt[0]);
    }
}

/* ------------------------------------------------------------------------ */
/* Counter-based dropout mask.                                               */
/* ------------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                       uint32_t out[4]) {
    /* Round multipliers and key increments as published for Philox4x32. */
    const uint32_t mult0 = 0xD2511F53u, mult1 = 0xCD9E8D57u;
    const uint32_t bump0 = 0x9E3779B9u, bump1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += bump0; k1 += bump1; }
        uint64_t prod0 = (uint64_t)mult0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)mult1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

uint32_t orc_dropout_threshold(float p) {
    return (uint32_t)floor((double)p * 65536.0 + 0.5);
}

void orc_dropout_keep(uint64_t seed, float p, int64_t rows, int64_t m,
                      uint8_t* keep) {
    orc_dropout_keep_rows(seed, p, 0, rows, m, keep);
}

void orc_dropout_keep_rows(uint64_t seed, float p, int64_t row0, int64_t rows, int64_t m,
                           uint8_t* keep) {
    uint32_t thr = orc_dropout_threshold(p);
    uint32_t key[2] = { (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32) };
    for (int64_t r = 0; r < rows; ++r) {
        uint64_t ur = (uint64_t)(row0 + r);
        for (int64_t j = 0; j < m; ++j) {
            uint64_t uj = (uint64_t)j;
            uint32_t ctr[4] = { (uint32_t)(uj >> 3), (uint32_t)(ur & 0xFFFFFFFFu),
                                (uint32_t)(ur >> 32), 0u };
            uint32_t w[4];
            orc_philox4x32_10(ctr, key, w);
            uint32_t k = (uint32_t)(uj & 7u);
            uint32_t u = (w[k >> 1] >> (16u * (k & 1u))) & 0xFFFFu;
            keep[r * m + j] = (uint8_t)(u >= thr ? 1 : 0);
        }
    }
}

void orc_bias_dropout_residual(const double* x, const double* bias,
                               const double* residual, const uint8_t* keep,
                               float p, int64_t rows, int64_t m, double* z) {
    double q = 1.0 - (double)p;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < m; ++j) {
            int64_t i = r * m + j;
            double t = x[i] + bias[j];
            double d = keep[i] ? t / q : 0.0;
            z[i] = residual[i] + d;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Backward ([L11] §2.1, §2.4).                                              */
/* ------------------------------------------------------------------------ */

void orc_dropout_residual_bwd(const double* dz, const uint8_t* keep, float p,
                              int64_t rows, int64_t m, double* dx,
                              double* dbias, double* sbias) {
    double q = 1.0 - (double)p;
    for (int64_t j = 0; j < m; ++j) {
        dbias[j] = 0.0;
        if (sbias) sbias[j] = 0.0;
    }
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < m; ++j) {
            int64_t i = r * m + j;
            dx[i] = keep[i] ? dz[i] / q : 0.0;
            dbias[j] += dx[i];
            if (sbias) sbias[j] += fabs(dx[i]);
        }
    }
}

void orc_ln_bwd_dx_hw4(const double* dy, const double* x, const double* gamma,
                       const double* mean, const double* rstd,
                       int64_t rows, int64_t m, double* dx) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* dyr = dy + r * m;
        const double* xr = x + r * m;
        double mu = mean[r], rs = rstd[r];
        double sum_g = 0.0, sum_gxhat = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double g = gamma[j] * dyr[j];
            double xhat = (xr[j] - mu) * rs;
            sum_g += g;
            sum_gxhat += g * xhat;
        }
        for (int64_t j = 0; j < m; ++j) {
            double g = gamma[j] * dyr[j];
            double xhat = (xr[j] - mu) * rs;
            dx[r * m + j] = rs * (g - (sum_g + xhat * sum_gxhat) / (double)m);
        }
    }
}

void orc_ln_bwd_dx_scale(const double* dy, const double* x, const double* gamma,
                         const double* mean, const double* rstd,
                         int64_t rows, int64_t m, double* scale) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* dyr = dy + r * m;
        const double* xr = x + r * m;
        double mu = mean[r], rs = rstd[r];
        double abs_g = 0.0, abs_gxhat = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double g = gamma[j] * dyr[j];
            double xhat = (xr[j] - mu) * rs;
            abs_g += fabs(g);
            abs_gxhat += fabs(g * xhat);
        }
        for (int64_t j = 0; j < m; ++j) {
            double g = gamma[j] * dyr[j];
            double xhat = (xr[j] - mu) * rs;
            scale[r * m + j] = rs * (fabs(g) + (abs_g + fabs(xhat) * abs_gxhat) / (double)m);
        }
    }
}

void orc_ln_bwd_dx_slides(const double* dy, const double* x,
                          const double* gamma, const double* mean,
                          const double* rstd, int64_t rows, int64_t m,
                          double* dx) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* dyr = dy + r * m;
        const double* xr = x + r * m;
        double mu = mean[r];
        double sigma = 1.0 / rstd[r];
        double sigma2 = sigma * sigma;
        double sigma3 = sigma2 * sigma;
        double sum_g = 0.0, sum_gx = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double g = gamma[j] * dyr[j];
            sum_g += g;
            sum_gx += g * xr[j];
        }
        for (int64_t j = 0; j < m; ++j) {
            double g = gamma[j] * dyr[j];
            double alpha = ((xr[j] - mu) * mu - sigma2) / ((double)m * sigma3);
            double beta = (mu - xr[j]) / ((double)m * sigma3);
            dx[r * m + j] = g / sigma + alpha * sum_g + beta * sum_gx;
        }
    }
}

void orc_ln_bwd_params(const double* dy, const double* x, const double* mean,
                       const double* rstd, int64_t rows, int64_t m,
                       double* dgamma, double* dbeta,
                       double* sgamma, double* sbeta) {
    for (int64_t j = 0; j < m; ++j) {
        dgamma[j] = 0.0;
        dbeta[j] = 0.0;
        if (sgamma) sgamma[j] = 0.0;
        if (sbeta) sbeta[j] = 0.0;
    }
    for (int64_t r = 0; r < rows; ++r) {
        double mu = mean[r], rs = rstd[r];
        for (int64_t j = 0; j < m; ++j) {
            double d = dy[r * m + j];
            double term = d * ((x[r * m + j] - mu) * rs);
            dgamma[j] += term;
            dbeta[j] += d;
            if (sgamma) sgamma[j] += fabs(term);
            if (sbeta) sbeta[j] += fabs(d);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Attention softmax ([L10] §4.1, [L11] §3).                                 */
/* ------------------------------------------------------------------------ */

void orc_attn_softmax_fwd(const double* x, const double* mask, int64_t rows_per_mask,
                          int64_t rows, int64_t m, double scale, int causal, double* y) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * m;
        const double* mr = mask ? mask + (r / rows_per_mask) * m : NULL;
        double* yr = y + r * m;
        int64_t q = r % m;
        /* scaled and masked scores, kept in y for the two passes below */
        double mx = -INFINITY;
        for (int64_t j = 0; j < m; ++j) {
            double t = scale * xr[j] + (mr ? mr[j] : 0.0);
            if (causal && j > q) t = -INFINITY;
            yr[j] = t;
            if (t > mx) mx = t;
        }
        if (mx == -INFINITY) {
            for (int64_t j = 0; j < m; ++j) yr[j] = 0.0;
            continue;
        }
        double sum = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            double e = exp(yr[j] - mx);
            yr[j] = e;
            sum += e;
        }
        for (int64_t j = 0; j < m; ++j) yr[j] = yr[j] / sum;
    }
}

void orc_attn_softmax_bwd(const double* dy, const double* y, const uint8_t* keep, float p,
                          int64_t rows, int64_t m, double scale, double* dx) {
    double q = 1.0 - (double)p;
    for (int64_t r = 0; r < rows; ++r) {
        const double* dyr = dy + r * m;
        const double* yr = y + r * m;
        double s = 0.0;
        for (int64_t j = 0; j < m; ++j) {
            int64_t i = r * m + j;
            double g = keep ? (keep[i] ? dyr[j] / q : 0.0) : dyr[j];
            dx[i] = g;               /* g, kept for the second pass */
            s += g * yr[j];
        }
        for (int64_t j = 0; j < m; ++j) {
            int64_t i = r * m + j;
            dx[i] = scale * yr[j] * (dx[i] - s);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm ([FP] §6: fused add + RMSNorm).                                   */
/* ------------------------------------------------------------------------ */

void orc_rmsnorm_fwd(const double* x, const double* gamma, int64_t rows, int64_t m,
                     double eps, double* y, double* rstd) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * m;
        double ss = 0.0;
        for (int64_t j = 0; j < m; ++j) ss += xr[j] * xr[j];
        double rs = 1.0 / sqrt(ss / (double)m + eps);
        rstd[r] = rs;
        for (int64_t j = 0; j < m; ++j) y[r * m + j] = gamma[j] * (xr[j] * rs);
    }
}

void orc_rmsnorm_bwd(const double* dy, const double* x, const double* gamma,
                     const double* rstd, int64_t rows, int64_t m, double* dx,
                     double* dgamma, double* sgamma) {
    for (int64_t j = 0; j < m; ++j) {
        dgamma[j] = 0.0;
        if (sgamma) sgamma[j] = 0.0;
    }
    for (int64_t r = 0; r < rows; ++r) {
        const double* dyr = dy + r * m;
        const double* xr = x + r * m;
        double rs = rstd[r];
        double b = 0.0;
        for (int64_t j = 0; j < m; ++j) b += gamma[j] * dyr[j] * (xr[j] * rs);
        for (int64_t j = 0; j < m; ++j) {
            double xhat = xr[j] * rs;
            dx[r * m + j] = rs * (gamma[j] * dyr[j] - xhat * b / (double)m);
            dgamma[j] += dyr[j] * xhat;
            if (sgamma) sgamma[j] += fabs(dyr[j] * xhat);
        }
    }
}


/* ------------------------------------------------------------------------ */
/* Cross-entropy with label smoothing ([L10] §5.2; [LLMC] §6.1).            */
/* ------------------------------------------------------------------------ */

void orc_cross_entropy(const double* x, const int64_t* labels, int64_t rows, int64_t V,
                       double alpha, double scale, double* loss, double* dx) {
    for (int64_t r = 0; r < rows; ++r) {
        const double* xr = x + r * V;
        double* dr = dx ? dx + r * V : NULL;
        const int64_t y = labels[r];
        if (y < 0 || y >= V) {
            const double v = y < 0 ? 0.0 : NAN;
            loss[r] = v;
            if (dr)
                for (int64_t j = 0; j < V; ++j) dr[j] = v;
            continue;
        }
        double mx = -INFINITY;
        for (int64_t j = 0; j < V; ++j)
            if (xr[j] > mx) mx = xr[j];
        double z = 0.0;
        for (int64_t j = 0; j < V; ++j) z += exp(xr[j] - mx);
        const double logz = log(z);
        double l = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            const double p = (j == y ? 1.0 - alpha : 0.0) + alpha / (double)V;
            const double logq = (xr[j] - mx) - logz;
            l -= p * logq;
            if (dr) dr[j] = scale * (exp(logq) - p);
        }
        loss[r] = l;
    }
}
