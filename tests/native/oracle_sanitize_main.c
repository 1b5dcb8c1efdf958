/* Drives the CPU oracle (oracle/gla_oracle.c) through every entry point on
 * small random problems, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py): both gate forms,
 * head sharing, document resets (a reset on the first and second token, one-token
 * documents), with and without h0 / dhT, T = 0 and T = 1, one and several threads,
 * d_v not a multiple of the thread column block.  Exits non-zero if a call fails
 * or an output is not finite; the sanitizers abort on any bad access. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gla_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv, int gate_vec,
                   const double *q, const double *k, const double *v, const double *g, const double *h0,
                   const int32_t *seg, double *o, double *hT, int nthreads);
int gla_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv, int gate_vec,
                   const double *q, const double *k, const double *v, const double *g, const double *h0,
                   const int32_t *seg, const double *dO, const double *dhT, double *dq, double *dk_out,
                   double *dv_out, double *dg, double *dh0, int nthreads);
int gla_oracle_bwd_per_head(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv,
                            int gate_vec, const double *q, const double *k, const double *v,
                            const double *g, const double *h0, const int32_t *seg, const double *dO,
                            const double *dhT, double *dq_h, double *dk_h, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double urand(void) {  /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / (double)(1ull << 52) - 1.0;
}
static double *arr(int64_t n, double scale) {
    double *x = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) x[i] = scale * urand();
    return x;
}
static int finite_all(const double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static int run_case(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv, int vec,
                    int with_states, int with_seg, int threads) {
    const int64_t nq = B * T * Hqk * dk, nv = B * T * H * dv, ng = B * T * H * (vec ? dk : 1);
    const int64_t ns = B * H * dk * dv;
    double *q = arr(nq, 0.3), *k = arr(nq, 0.3), *v = arr(nv, 1.0), *g = arr(ng, 0.5);
    for (int64_t i = 0; i < ng; ++i) g[i] = -fabs(g[i]);
    double *h0 = with_states ? arr(ns, 0.1) : NULL, *dhT = with_states ? arr(ns, 1.0) : NULL;
    double *dO = arr(nv, 1.0), *o = arr(nv, 0.0), *hT = arr(ns, 0.0);
    double *dq = arr(nq, 0.0), *dk_ = arr(nq, 0.0), *dv_ = arr(nv, 0.0), *dg = arr(ng, 0.0);
    double *dh0 = arr(ns, 0.0);
    double *dqh = arr(B * T * H * dk, 0.0), *dkh = arr(B * T * H * dk, 0.0);
    int32_t *seg = NULL;
    if (with_seg) {
        seg = (int32_t *)malloc((size_t)(B * T > 0 ? B * T : 1) * sizeof(int32_t));
        for (int64_t b = 0; b < B; ++b) {
            int32_t id = 0;
            for (int64_t t = 0; t < T; ++t) {
                if (t == 1 || t == 2 || (t > 2 && urand() > 0.8)) ++id;  /* one-token documents */
                seg[b * T + t] = id;
            }
        }
    }
    int bad = 0;
    if (gla_oracle_fwd(B, T, H, Hqk, dk, dv, vec, q, k, v, g, h0, seg, o, hT, threads)) bad |= 1;
    if (gla_oracle_bwd(B, T, H, Hqk, dk, dv, vec, q, k, v, g, h0, seg, dO, dhT, dq, dk_, dv_, dg, dh0,
                       threads)) bad |= 2;
    if (gla_oracle_bwd_per_head(B, T, H, Hqk, dk, dv, vec, q, k, v, g, h0, seg, dO, dhT, dqh, dkh,
                                threads)) bad |= 4;
    if (!finite_all(o, nv) || !finite_all(hT, ns) || !finite_all(dq, nq) || !finite_all(dk_, nq) ||
        !finite_all(dv_, nv) || !finite_all(dg, ng) || !finite_all(dh0, ns) ||
        !finite_all(dqh, B * T * H * dk) || !finite_all(dkh, B * T * H * dk)) bad |= 8;
    if (bad)
        fprintf(stderr, "case B%lld T%lld H%lld Hqk%lld dk%lld dv%lld vec%d states%d seg%d threads%d: %d\n",
                (long long)B, (long long)T, (long long)H, (long long)Hqk, (long long)dk, (long long)dv,
                vec, with_states, with_seg, threads, bad);
    free(q); free(k); free(v); free(g); free(h0); free(dhT); free(dO); free(o); free(hT);
    free(dq); free(dk_); free(dv_); free(dg); free(dh0); free(dqh); free(dkh); free(seg);
    return bad;
}

int main(void) {
    int bad = 0, n = 0;
    for (int vec = 0; vec < 2; ++vec)
        for (int states = 0; states < 2; ++states)
            for (int segs = 0; segs < 2; ++segs) {
                const int64_t shapes[][6] = {
                    {2, 37, 4, 2, 8, 6}, {1, 1, 2, 2, 4, 4}, {2, 0, 2, 1, 4, 4}, {1, 70, 3, 1, 5, 9}};
                for (int s = 0; s < 4; ++s)
                    for (int th = 1; th <= 3; th += 2) {
                        const int64_t *x = shapes[s];
                        bad |= run_case(x[0], x[1], x[2], x[3], x[4], x[5], vec, states, segs, th);
                        ++n;
                    }
            }
    printf("%d oracle cases, %s\n", n, bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}
