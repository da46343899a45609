/* Host-only sanitizer run of the fp64 oracle (test infrastructure): the oracle's C
 * source is compiled into this driver with AddressSanitizer and
 * UndefinedBehaviorSanitizer, and every entry point runs on ragged packed
 * sequences (empty, one-token and sub-chunk-crossing lengths), with and without
 * initial states, conv states, bias and each flag.  A planted closed form keeps the
 * run meaningful: with beta = 0 nothing is written, so the final state is the
 * initial one decayed row by row by exp(sum of g), g = lb * sigmoid(a). */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/kda_oracle.c"

static double urand(unsigned long long *s) {
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((double)(*s >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}

static double *fill(size_t n, unsigned long long *s, double scale) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = scale * urand(s);
    return p;
}

int main(void) {
    const int32_t lens[] = {0, 1, 3, 17, 64, 65, 0, 130};
    const int N = (int)(sizeof(lens) / sizeof(lens[0]));
    const int H = 2, D = 128, CC = 3 * H * D;
    int32_t cu[sizeof(lens) / sizeof(lens[0]) + 1];
    cu[0] = 0;
    for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + lens[n];
    const int64_t T = cu[N];
    unsigned long long seed = 12345;
    double *q = fill((size_t)T * H * D, &seed, 1.0), *k = fill((size_t)T * H * D, &seed, 1.0);
    double *v = fill((size_t)T * H * D, &seed, 1.0), *a = fill((size_t)T * H * D, &seed, 2.0);
    double *beta = fill((size_t)T * H, &seed, 0.5);
    for (int64_t i = 0; i < T * H; ++i) beta[i] += 0.5;
    double *w = fill((size_t)CC * 4, &seed, 0.5), *b = fill(CC, &seed, 0.1);
    double *cs_in = fill((size_t)N * 3 * CC, &seed, 1.0), *s_in = fill((size_t)N * H * D * D, &seed, 0.1);
    double *o = (double *)calloc((size_t)T * H * D + 1, sizeof(double));
    double *s_out = (double *)calloc((size_t)N * H * D * D, sizeof(double));
    double *cs_out = (double *)calloc((size_t)N * 3 * CC, sizeof(double));
    const unsigned flag_sets[] = {0u, 1u, 2u, 4u, 7u};
    for (int f = 0; f < 5; ++f)
        for (int with_state = 0; with_state < 2; ++with_state) {
            kda_oracle_prefill(N, H, D, D, cu, q, k, v, a, beta, w, with_state ? b : NULL,
                               with_state ? cs_in : NULL, cs_out, with_state ? s_in : NULL, s_out, o,
                               1.0 / sqrt(128.0), -5.0, flag_sets[f], 1);
        }
    /* beta = 0: the final state is the decayed initial state */
    double *zero = (double *)calloc((size_t)T * H + 1, sizeof(double));
    kda_oracle_prefill(N, H, D, D, cu, q, k, v, a, zero, w, NULL, NULL, cs_out, s_in, s_out, o,
                       1.0 / sqrt(128.0), -5.0, 0u, 1);
    double worst = 0.0;
    for (int n = 0; n < N; ++n)
        for (int h = 0; h < H; ++h)
            for (int r = 0; r < D; ++r) {
                double gs = 0.0;
                for (int t = cu[n]; t < cu[n + 1]; ++t) {
                    const double x = a[((size_t)t * H + h) * D + r];
                    gs += -5.0 / (1.0 + exp(-x));
                }
                for (int c = 0; c < D; ++c) {
                    const size_t at = (((size_t)n * H + h) * D + r) * D + c;
                    const double e = fabs(s_out[at] - s_in[at] * exp(gs));
                    worst = e > worst ? e : worst;
                }
            }
    if (worst > 1e-12) {
        fprintf(stderr, "beta = 0 closed form off by %g\n", worst);
        return 1;
    }
    double *y = (double *)calloc((size_t)T * CC + 1, sizeof(double));
    kda_oracle_short_conv(q, y, T, CC / 3, w, b, cs_in, cs_out, cu, N, 1, 1);
    double *sd = fill((size_t)N * H * D * D, &seed, 0.1), *csd = fill((size_t)N * 3 * CC, &seed, 1.0);
    double *od = (double *)calloc((size_t)N * H * D, sizeof(double));
    kda_oracle_decode(N, H, D, D, q, k, v, a, beta, w, b, csd, sd, od, 1.0 / sqrt(128.0), -5.0, 0u, 1);
    free(q); free(k); free(v); free(a); free(beta); free(w); free(b); free(cs_in); free(s_in);
    free(o); free(s_out); free(cs_out); free(zero); free(y); free(sd); free(csd); free(od);
    printf("oracle sanitizer run ok (beta = 0 closed form within %g)\n", worst);
    return 0;
}
