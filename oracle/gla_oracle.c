/*
 * gla_oracle.c -- fp64, token-by-token CPU oracle for the gated linear-attention
 * recurrence.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP library.
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg may build, load or call it; the product path never does.  It shares no
 * code, header or table with the HIP library.
 *
 * What it computes (per batch row b and head h, G = H / H_qk heads share one
 * q/k head, h_qk = floor(h / G)):
 *
 *   S_{-1} = h0[b,h]   (zeros if absent)
 *   for t = 0 .. T-1:
 *       if t > 0 and seg[b,t] != seg[b,t-1]:  S = 0          (document reset)
 *       else:                                  S = diag(exp g_t) S
 *       S += k_t v_t^T
 *       o_t = S^T q_t
 *   hT = S
 *
 * The recurrence S_t = diag(alpha_t) S_{t-1} + k_t v_t^T with o_t = S_t^T q_t
 * is the one written on the FLAT page ("FLAT: Flash Linear Attention on TPUs",
 * section Linear Attention > Forward Recurrence, with the gate table's notation
 * F_t = prod_{s<=t} f_s: a scalar gate for Mamba-2, a per-key-channel vector
 * gate for GLA).  The reset rule follows the JLA page ("JLA: JAX Linear
 * Attention", the paragraph on segment_ids): a packed row behaves exactly as
 * its documents run one by one, the first one from h0 and the rest from zero.
 * g is the natural-log gate, alpha_t = exp(g_t); at a reset token it is unused.
 *
 * Backward (FLAT page, Linear Attention > Backward Recurrence: the state
 * gradient runs backwards in time with the same form as the forward, the gate
 * scales it at every step, and grad_{f_t} = (grad_{H_t} (.) H_{t-1}) 1_V, so
 * grad_{log f_t} = f_t grad_{f_t}).  With dS the gradient of S_t:
 *
 *   dS = dhT (zeros if absent)
 *   for t = T-1 .. 0:
 *       dS += q_t dO_t^T
 *       dq_t = S_t dO_t ;  dk_t = dS v_t ;  dv_t = dS^T k_t
 *       if t is a reset:  dg_t = 0 ;  dS = 0
 *       else:             dg_t = alpha_t (.) rowsum(dS (.) S_{t-1}) ;  dS = diag(alpha_t) dS
 *                         (scalar gate: the sum runs over every entry)
 *   dh0 = dS
 *   dq, dk of a shared q/k head = sum over the G heads that read it.
 *
 * States for the reverse sweep come from checkpoints every CKPT tokens and a
 * forward recompute inside each span.  Work is split over (b, h, block of
 * d_v columns): the columns of S evolve independently, so each task owns its
 * columns of o, hT, dv, dh0 outright and writes partial dq, dk, dg that are
 * summed afterwards in a fixed order (results do not depend on thread count).
 *
 * Layouts (row-major, contiguous):
 *   q, k, dq, dk : [B, T, H_qk, d_k]      v, o, dO, dv : [B, T, H, d_v]
 *   g, dg        : [B, T, H] (scalar) or [B, T, H, d_k] (vector)
 *   h0, hT, dhT, dh0 : [B, H, d_k, d_v]   seg : [B, T] int32
 * Return value: 0 on success, -1 on bad sizes, -2 on allocation failure.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

typedef struct {
    int64_t B, T, H, Hqk, dk, dv;
    int vec;
    const double *q, *k, *v, *g, *h0, *dO, *dhT;
    const int32_t *seg;
    double *o, *hT;
    /* backward partials: [njb][B][T][H][dk] and [njb][B][T][H](x dk) */
    double *dq_part, *dk_part, *dg_part;
    double *dvo, *dh0;
    int64_t jb_width, njb;
    int64_t ntasks;
    int64_t next; /* next task index, guarded by mu */
    int failed;
    pthread_mutex_t mu;
} job_t;

static int64_t ntask_of(const job_t *J) { return J->B * J->H * J->njb; }

static int is_reset(const job_t *J, int64_t b, int64_t t) {
    return J->seg != NULL && t > 0 && J->seg[b * J->T + t] != J->seg[b * J->T + t - 1];
}

/* alpha_t for key channel c */
static double alpha_at(const job_t *J, int64_t b, int64_t t, int64_t h, int64_t c) {
    if (J->vec) return exp(J->g[((b * J->T + t) * J->H + h) * J->dk + c]);
    return exp(J->g[(b * J->T + t) * J->H + h]);
}

/* One token of the forward recurrence on columns [j0, j1) of S (S is dk x nj). */
static void step_forward(const job_t *J, int64_t b, int64_t t, int64_t h, int64_t j0,
                         int64_t nj, double *S) {
    const int64_t G = J->H / J->Hqk, hq = h / G;
    const double *kt = J->k + ((b * J->T + t) * J->Hqk + hq) * J->dk;
    const double *vt = J->v + ((b * J->T + t) * J->H + h) * J->dv + j0;
    const int reset = is_reset(J, b, t);
    for (int64_t c = 0; c < J->dk; ++c) {
        double *row = S + c * nj;
        if (reset) {
            for (int64_t j = 0; j < nj; ++j) row[j] = 0.0;
        } else {
            const double a = alpha_at(J, b, t, h, c);
            for (int64_t j = 0; j < nj; ++j) row[j] *= a;
        }
        for (int64_t j = 0; j < nj; ++j) row[j] += kt[c] * vt[j];
    }
}

static void load_h0(const job_t *J, int64_t b, int64_t h, int64_t j0, int64_t nj, double *S) {
    for (int64_t c = 0; c < J->dk; ++c)
        for (int64_t j = 0; j < nj; ++j)
            S[c * nj + j] = J->h0 ? J->h0[((b * J->H + h) * J->dk + c) * J->dv + j0 + j] : 0.0;
}

static void task_split(const job_t *J, int64_t task, int64_t *b, int64_t *h, int64_t *jb) {
    *jb = task % J->njb;
    int64_t bh = task / J->njb;
    *h = bh % J->H;
    *b = bh / J->H;
}

static int fwd_task(job_t *J, int64_t task) {
    int64_t b, h, jb;
    task_split(J, task, &b, &h, &jb);
    const int64_t j0 = jb * J->jb_width;
    const int64_t nj = (j0 + J->jb_width <= J->dv) ? J->jb_width : J->dv - j0;
    const int64_t G = J->H / J->Hqk, hq = h / G;
    double *S = (double *)malloc(sizeof(double) * J->dk * nj);
    if (!S) return -2;
    load_h0(J, b, h, j0, nj, S);
    for (int64_t t = 0; t < J->T; ++t) {
        step_forward(J, b, t, h, j0, nj, S);
        const double *qt = J->q + ((b * J->T + t) * J->Hqk + hq) * J->dk;
        double *ot = J->o + ((b * J->T + t) * J->H + h) * J->dv + j0;
        for (int64_t j = 0; j < nj; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < J->dk; ++c) acc += S[c * nj + j] * qt[c];
            ot[j] = acc;
        }
    }
    if (J->hT)
        for (int64_t c = 0; c < J->dk; ++c)
            for (int64_t j = 0; j < nj; ++j)
                J->hT[((b * J->H + h) * J->dk + c) * J->dv + j0 + j] = S[c * nj + j];
    free(S);
    return 0;
}

static int bwd_task(job_t *J, int64_t task) {
    int64_t b, h, jb;
    task_split(J, task, &b, &h, &jb);
    const int64_t T = J->T, dk = J->dk, dv = J->dv, H = J->H;
    const int64_t j0 = jb * J->jb_width;
    const int64_t nj = (j0 + J->jb_width <= dv) ? J->jb_width : dv - j0;
    const int64_t G = H / J->Hqk, hq = h / G;
    const int64_t nspan = (T + CKPT - 1) / CKPT;
    const int64_t sz = dk * nj;
    double *ckpt = (double *)malloc(sizeof(double) * sz * (nspan > 0 ? nspan : 1));
    double *states = (double *)malloc(sizeof(double) * sz * CKPT);
    double *dS = (double *)malloc(sizeof(double) * sz);
    double *S = (double *)malloc(sizeof(double) * sz);
    if (!ckpt || !states || !dS || !S) {
        free(ckpt); free(states); free(dS); free(S);
        return -2;
    }
    /* forward sweep: ckpt[n] = state entering token n*CKPT */
    load_h0(J, b, h, j0, nj, S);
    for (int64_t t = 0; t < T; ++t) {
        if (t % CKPT == 0) memcpy(ckpt + (t / CKPT) * sz, S, sizeof(double) * sz);
        step_forward(J, b, t, h, j0, nj, S);
    }
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < nj; ++j)
            dS[c * nj + j] = J->dhT ? J->dhT[((b * H + h) * dk + c) * dv + j0 + j] : 0.0;

    double *dqp = J->dq_part + jb * (J->B * T * H * dk);
    double *dkp = J->dk_part + jb * (J->B * T * H * dk);
    const int64_t gw = J->vec ? dk : 1;
    double *dgp = J->dg_part + jb * (J->B * T * H * gw);

    for (int64_t n = nspan - 1; n >= 0; --n) {
        const int64_t t0 = n * CKPT, t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
        memcpy(S, ckpt + n * sz, sizeof(double) * sz);
        for (int64_t t = t0; t < t1; ++t) {
            step_forward(J, b, t, h, j0, nj, S);
            memcpy(states + (t - t0) * sz, S, sizeof(double) * sz);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double *St = states + (t - t0) * sz;
            const double *Sp = (t > t0) ? states + (t - t0 - 1) * sz : ckpt + n * sz;
            const double *qt = J->q + ((b * T + t) * J->Hqk + hq) * dk;
            const double *kt = J->k + ((b * T + t) * J->Hqk + hq) * dk;
            const double *vt = J->v + ((b * T + t) * H + h) * dv + j0;
            const double *dot = J->dO + ((b * T + t) * H + h) * dv + j0;
            double *dqt = dqp + ((b * T + t) * H + h) * dk;
            double *dkt = dkp + ((b * T + t) * H + h) * dk;
            double *dgt = dgp + ((b * T + t) * H + h) * gw;
            double *dvt = J->dvo + ((b * T + t) * H + h) * dv + j0;
            /* gradient of S_t: add this token's readout */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < nj; ++j) dS[c * nj + j] += qt[c] * dot[j];
            for (int64_t c = 0; c < dk; ++c) {
                double aq = 0.0, ak = 0.0;
                for (int64_t j = 0; j < nj; ++j) {
                    aq += St[c * nj + j] * dot[j];
                    ak += dS[c * nj + j] * vt[j];
                }
                dqt[c] = aq;
                dkt[c] = ak;
            }
            for (int64_t j = 0; j < nj; ++j) {
                double a = 0.0;
                for (int64_t c = 0; c < dk; ++c) a += dS[c * nj + j] * kt[c];
                dvt[j] = a;
            }
            if (is_reset(J, b, t)) {
                for (int64_t i = 0; i < gw; ++i) dgt[i] = 0.0;
                for (int64_t i = 0; i < sz; ++i) dS[i] = 0.0;
            } else {
                double tot = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    const double a = alpha_at(J, b, t, h, c);
                    double r = 0.0;
                    for (int64_t j = 0; j < nj; ++j) r += dS[c * nj + j] * Sp[c * nj + j];
                    if (J->vec) dgt[c] = a * r;
                    else tot += a * r;
                    for (int64_t j = 0; j < nj; ++j) dS[c * nj + j] *= a;
                }
                if (!J->vec) dgt[0] = tot;
            }
        }
    }
    if (J->dh0)
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < nj; ++j)
                J->dh0[((b * H + h) * dk + c) * dv + j0 + j] = dS[c * nj + j];
    free(ckpt); free(states); free(dS); free(S);
    return 0;
}

typedef struct { job_t *J; int bwd; } worker_arg;

static void *worker(void *p) {
    worker_arg *W = (worker_arg *)p;
    job_t *J = W->J;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t task = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (task >= J->ntasks) break;
        int rc = W->bwd ? bwd_task(J, task) : fwd_task(J, task);
        if (rc) {
            pthread_mutex_lock(&J->mu);
            J->failed = rc;
            pthread_mutex_unlock(&J->mu);
        }
    }
    return NULL;
}

static int run(job_t *J, int bwd, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    J->ntasks = ntask_of(J);
    J->next = 0;
    J->failed = 0;
    pthread_mutex_init(&J->mu, NULL);
    worker_arg W = {J, bwd};
    if (nthreads == 1 || J->ntasks <= 1) {
        worker(&W);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
        if (!th) { pthread_mutex_destroy(&J->mu); return -2; }
        int started = 0;
        for (int i = 0; i < nthreads; ++i)
            if (pthread_create(&th[i], NULL, worker, &W) == 0) ++started;
        if (started == 0) worker(&W);
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J->mu);
    return J->failed;
}

static int check_sizes(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv) {
    if (B < 0 || T < 0 || H < 1 || Hqk < 1 || dk < 1 || dv < 1) return -1;
    if (H % Hqk) return -1;
    return 0;
}

/* Column-block width: whole d_v when there are enough (b, h) tasks. */
static int64_t pick_jb(int64_t B, int64_t H, int64_t dv, int nthreads) {
    int64_t w = dv;
    while (B * H * (dv / w) < nthreads && w > 16 && w % 2 == 0) w /= 2;
    return w;
}

int gla_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv,
                   int gate_vec, const double *q, const double *k, const double *v,
                   const double *g, const double *h0, const int32_t *seg, double *o,
                   double *hT, int nthreads) {
    if (check_sizes(B, T, H, Hqk, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.Hqk = Hqk; J.dk = dk; J.dv = dv; J.vec = gate_vec != 0;
    J.q = q; J.k = k; J.v = v; J.g = g; J.h0 = h0; J.seg = seg; J.o = o; J.hT = hT;
    J.jb_width = pick_jb(B, H, dv, nthreads);
    J.njb = (dv + J.jb_width - 1) / J.jb_width;
    return run(&J, 0, nthreads);
}

int gla_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk, int64_t dv,
                   int gate_vec, const double *q, const double *k, const double *v,
                   const double *g, const double *h0, const int32_t *seg, const double *dO,
                   const double *dhT, double *dq, double *dk_out, double *dv_out, double *dg,
                   double *dh0, int nthreads) {
    if (check_sizes(B, T, H, Hqk, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.Hqk = Hqk; J.dk = dk; J.dv = dv; J.vec = gate_vec != 0;
    J.q = q; J.k = k; J.v = v; J.g = g; J.h0 = h0; J.seg = seg; J.dO = dO; J.dhT = dhT;
    J.dvo = dv_out; J.dh0 = dh0;
    J.jb_width = pick_jb(B, H, dv, nthreads);
    J.njb = (dv + J.jb_width - 1) / J.jb_width;
    const int64_t gw = J.vec ? dk : 1;
    const int64_t nqk = B * T * H * dk;
    J.dq_part = (double *)calloc((size_t)(J.njb * nqk > 0 ? J.njb * nqk : 1), sizeof(double));
    J.dk_part = (double *)calloc((size_t)(J.njb * nqk > 0 ? J.njb * nqk : 1), sizeof(double));
    J.dg_part = (double *)calloc((size_t)(J.njb * B * T * H * gw > 0 ? J.njb * B * T * H * gw : 1),
                                 sizeof(double));
    if (!J.dq_part || !J.dk_part || !J.dg_part) {
        free(J.dq_part); free(J.dk_part); free(J.dg_part);
        return -2;
    }
    int rc = run(&J, 1, nthreads);
    if (rc == 0) {
        const int64_t G = H / Hqk;
        /* fixed-order reduction over column blocks, then over the heads of a group */
        for (int64_t b = 0; b < B; ++b)
            for (int64_t t = 0; t < T; ++t) {
                for (int64_t hq = 0; hq < Hqk; ++hq)
                    for (int64_t c = 0; c < dk; ++c) {
                        double sq = 0.0, sk = 0.0;
                        for (int64_t h = hq * G; h < (hq + 1) * G; ++h)
                            for (int64_t jb = 0; jb < J.njb; ++jb) {
                                const int64_t idx = jb * nqk + ((b * T + t) * H + h) * dk + c;
                                sq += J.dq_part[idx];
                                sk += J.dk_part[idx];
                            }
                        dq[((b * T + t) * Hqk + hq) * dk + c] = sq;
                        dk_out[((b * T + t) * Hqk + hq) * dk + c] = sk;
                    }
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t i = 0; i < gw; ++i) {
                        double s = 0.0;
                        for (int64_t jb = 0; jb < J.njb; ++jb)
                            s += J.dg_part[jb * (B * T * H * gw) + ((b * T + t) * H + h) * gw + i];
                        dg[((b * T + t) * H + h) * gw + i] = s;
                    }
            }
    }
    free(J.dq_part); free(J.dk_part); free(J.dg_part);
    return rc;
}

/* Per-head (pre-group-sum) dq and dk, needed by checks of the gate-gradient
 * identity, which holds head by head.  Same sweep as gla_oracle_bwd; dq_h and
 * dk_h are [B, T, H, d_k]. */
int gla_oracle_bwd_per_head(int64_t B, int64_t T, int64_t H, int64_t Hqk, int64_t dk,
                            int64_t dv, int gate_vec, const double *q, const double *k,
                            const double *v, const double *g, const double *h0,
                            const int32_t *seg, const double *dO, const double *dhT,
                            double *dq_h, double *dk_h, int nthreads) {
    if (check_sizes(B, T, H, Hqk, dk, dv)) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.B = B; J.T = T; J.H = H; J.Hqk = Hqk; J.dk = dk; J.dv = dv; J.vec = gate_vec != 0;
    J.q = q; J.k = k; J.v = v; J.g = g; J.h0 = h0; J.seg = seg; J.dO = dO; J.dhT = dhT;
    J.jb_width = pick_jb(B, H, dv, nthreads);
    J.njb = (dv + J.jb_width - 1) / J.jb_width;
    const int64_t gw = J.vec ? dk : 1;
    const int64_t nqk = B * T * H * dk;
    J.dvo = (double *)calloc((size_t)(B * T * H * dv > 0 ? B * T * H * dv : 1), sizeof(double));
    J.dq_part = (double *)calloc((size_t)(J.njb * nqk > 0 ? J.njb * nqk : 1), sizeof(double));
    J.dk_part = (double *)calloc((size_t)(J.njb * nqk > 0 ? J.njb * nqk : 1), sizeof(double));
    J.dg_part = (double *)calloc((size_t)(J.njb * B * T * H * gw > 0 ? J.njb * B * T * H * gw : 1),
                                 sizeof(double));
    if (!J.dvo || !J.dq_part || !J.dk_part || !J.dg_part) {
        free(J.dvo); free(J.dq_part); free(J.dk_part); free(J.dg_part);
        return -2;
    }
    int rc = run(&J, 1, nthreads);
    if (rc == 0)
        for (int64_t i = 0; i < nqk; ++i) {
            double sq = 0.0, sk = 0.0;
            for (int64_t jb = 0; jb < J.njb; ++jb) {
                sq += J.dq_part[jb * nqk + i];
                sk += J.dk_part[jb * nqk + i];
            }
            dq_h[i] = sq;
            dk_h[i] = sk;
        }
    free(J.dvo); free(J.dq_part); free(J.dk_part); free(J.dg_part);
    return rc;
}
