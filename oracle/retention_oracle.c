/*
 * Retention oracle: a plain, slow, fp64 CPU implementation of multi-scale retention.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * this library. The GPU library neither links nor calls it, and this file includes none of its headers.
 *
 * What is computed (sources: "Hybrid Architectures: RetNet and the Three Computation Paradigms",
 * sections 2-7; the RetNet paper summary, Eq. 5, 6 and 7):
 *   - rotation of q and k by the position angle p*theta_i on dimension pairs (2i, 2i+1);
 *   - the parallel form   O = (Q K^T (.) D) V,  D[n][m] = gamma^(n-m) for n >= m, else 0;
 *   - the recurrent form  S_n = gamma S_{n-1} + k_n^T v_n,  o_n = q_n S_n  (update, then read);
 *   - the chunkwise form  O_[i] = (Q_[i] K_[i]^T (.) D) V_[i] + (Q_[i] R_{i-1}) (.) xi,
 *                         R_i = gamma^L R_{i-1} + K_[i]^T (V_[i] (.) zeta);
 *   - the parallel form with the retention score normalizations (blog section 8.5; paper summary,
 *     "Retention Score Normalization"): QK^T / sqrt(d_k), D~ and R~; and the recurrent and chunkwise forms
 *     with the same normalizations, carried through the decayed key sum z (reading below);
 *   - the multi-scale retention epilogue (blog sections 8.4 and 9.1; paper summary, "Gating mechanism"):
 *     y = swish(g) (.) GroupNorm_h(o), with g = X W_G given;
 *   - the gradients of the recurrent form from a zero state (the pages train with the chunkwise form, paper
 *     summary "Overall RetNet Architecture and Training/Inference Protocol"), by the adjoint of the scan:
 *     dq'_n = S_n dO_n, G_n = gamma G_{n+1} + q'_n^T dO_n, dk'_n = G_n v_n, dv_n = G_n^T k'_n, then dq, dk
 *     rotated back by the transpose rotation.
 *
 * Readings where the pages leave a step open (each is also listed in the design notes):
 *   - the rotation turns pair (x_{2i}, x_{2i+1}) of BOTH q and k by +p*theta_i, then a real dot product
 *     is taken; this equals Re( sum_i qc_i * conj(kc_i) * e^{i (n-m) theta_i} ) with qc_i = q_{2i} + i q_{2i+1},
 *     the conjugate-transpose form of the paper summary's unrolled equation;
 *   - the absolute position of token n is p = pos0 + n;
 *   - a tail chunk of length L < C uses gamma^L for the carry and zeta_l = gamma^(L-1-l);
 *   - state_in (when given) is the state before token 0; the parallel form takes none.
 *
 * Layouts (row-major, fp64): q, k [B][N][H][dk]; v, o [B][N][H][dv]; state [B][H][dk][dv]; gamma [H];
 * theta [dk/2] or NULL for no rotation. (b, h) pairs are independent and are spread over threads; the
 * arithmetic for one pair is the same whatever the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------------ */
/* Rotation (blog section 6.6-6.8; paper summary, parallel representation: Q = (X W_Q) (.) Theta).   */
/* ------------------------------------------------------------------------------------------------ */

/* Gather row n of head h from a [B][N][H][d] tensor into dst[d], rotated to absolute position p. */
static void gather_rotated(const double* x, double* dst, int N, int H, int d, int b, int n, int h,
                           const double* theta, long long p) {
    const double* src = x + (((size_t)b * N + n) * H + h) * (size_t)d;
    if (!theta) {
        memcpy(dst, src, sizeof(double) * (size_t)d);
        return;
    }
    for (int i = 0; i < d / 2; ++i) {
        double phi = (double)p * theta[i];
        double c = cos(phi), s = sin(phi);
        double x0 = src[2 * i], x1 = src[2 * i + 1];
        dst[2 * i] = x0 * c - x1 * s;
        dst[2 * i + 1] = x0 * s + x1 * c;
    }
}

static void gather_plain(const double* x, double* dst, int N, int H, int d, int b, int n, int h) {
    memcpy(dst, x + (((size_t)b * N + n) * H + h) * (size_t)d, sizeof(double) * (size_t)d);
}

static double dot(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += a[i] * b[i];
    return s;
}

/* One (b, h) sequence, copied out and rotated: Qr, Kr [N][dk], Vh [N][dv]. */
typedef struct {
    double *Qr, *Kr, *Vh;
} head_seq;

static int load_head(head_seq* hs, const double* q, const double* k, const double* v, int N, int H, int dk,
                     int dv, int b, int h, const double* theta, long long pos0) {
    hs->Qr = (double*)malloc(sizeof(double) * (size_t)N * dk + 8);
    hs->Kr = (double*)malloc(sizeof(double) * (size_t)N * dk + 8);
    hs->Vh = (double*)malloc(sizeof(double) * (size_t)N * dv + 8);
    if (!hs->Qr || !hs->Kr || !hs->Vh) return -1;
    for (int n = 0; n < N; ++n) {
        gather_rotated(q, hs->Qr + (size_t)n * dk, N, H, dk, b, n, h, theta, pos0 + n);
        gather_rotated(k, hs->Kr + (size_t)n * dk, N, H, dk, b, n, h, theta, pos0 + n);
        gather_plain(v, hs->Vh + (size_t)n * dv, N, H, dv, b, n, h);
    }
    return 0;
}

static void free_head(head_seq* hs) {
    free(hs->Qr);
    free(hs->Kr);
    free(hs->Vh);
}

static double* out_row(double* o, int N, int H, int dv, int b, int n, int h) {
    return o + (((size_t)b * N + n) * H + h) * (size_t)dv;
}

/* ------------------------------------------------------------------------------------------------ */
/* Thread fan-out over (b, h) pairs.                                                                 */
/* ------------------------------------------------------------------------------------------------ */

typedef struct {
    const double *q, *k, *v, *gamma, *theta, *s_in, *z_in;
    double *o, *s_out, *z_out;
    const long long* rows;
    int nrows;
    int B, N, H, dk, dv, chunk;
    long long pos0;
    int form; /* 0 parallel, 1 recurrent, 2 chunkwise, 3 parallel rows, 4 normalized parallel,
                 6 normalized recurrent, 7 normalized chunkwise */
    int norm; /* normalized forms: ORC_NORM_* flags */
    const double* dout; /* gradients (form 5): dO [B][N][H][dv] in, dq, dk, dv out */
    double *dq, *dk_, *dv_;
    int nthreads, tid;
    int status;
} job;

static int form_parallel(job* J, int b, int h);
static int form_recurrent(job* J, int b, int h);
static int form_chunkwise(job* J, int b, int h);
static int form_parallel_rows(job* J, int b, int h);
static int form_parallel_norm(job* J, int b, int h);
static int form_grad(job* J, int b, int h);
static int form_recurrent_norm(job* J, int b, int h);
static int form_chunkwise_norm(job* J, int b, int h);

static void* worker(void* arg) {
    job* J = (job*)arg;
    int pairs = J->B * J->H;
    for (int u = J->tid; u < pairs; u += J->nthreads) {
        int b = u / J->H, h = u % J->H, rc = 0;
        switch (J->form) {
            case 0: rc = form_parallel(J, b, h); break;
            case 1: rc = form_recurrent(J, b, h); break;
            case 2: rc = form_chunkwise(J, b, h); break;
            case 4: rc = form_parallel_norm(J, b, h); break;
            case 5: rc = form_grad(J, b, h); break;
            case 6: rc = form_recurrent_norm(J, b, h); break;
            case 7: rc = form_chunkwise_norm(J, b, h); break;
            default: rc = form_parallel_rows(J, b, h); break;
        }
        if (rc) J->status = rc;
    }
    return NULL;
}

static int run(job proto) {
    int pairs = proto.B * proto.H;
    int nt = proto.nthreads < 1 ? 1 : proto.nthreads;
    if (nt > pairs) nt = pairs;
    if (nt > 256) nt = 256;
    job jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nt; ++t) {
        jobs[t] = proto;
        jobs[t].nthreads = nt;
        jobs[t].tid = t;
        jobs[t].status = 0;
    }
    for (int t = 1; t < nt; ++t)
        if (pthread_create(&th[t], NULL, worker, &jobs[t])) return -2;
    worker(&jobs[0]);
    for (int t = 1; t < nt; ++t) pthread_join(th[t], NULL);
    for (int t = 0; t < nt; ++t)
        if (jobs[t].status) return jobs[t].status;
    return 0;
}

static int check_args(int B, int N, int H, int dk, int dv, const double* gamma, const double* theta) {
    if (B <= 0 || N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !gamma) return -1;
    if (theta && (dk % 2)) return -1;
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Parallel form: the definition. o_n = sum_{m<=n} gamma^(n-m) (q_n . k_m) v_m                       */
/* (blog sections 2.2 and 4.2-4.3; paper summary Eq. 5).                                            */
/* ------------------------------------------------------------------------------------------------ */

static void parallel_row(const head_seq* hs, int dk, int dv, double gamma, int n, double* o) {
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int m = 0; m <= n; ++m) {
        double D = pow(gamma, (double)(n - m)); /* D[n][m], n >= m */
        double w = dot(hs->Qr + (size_t)n * dk, hs->Kr + (size_t)m * dk, dk) * D;
        const double* vm = hs->Vh + (size_t)m * dv;
        for (int j = 0; j < dv; ++j) o[j] += w * vm[j];
    }
}

static int form_parallel(job* J, int b, int h) {
    head_seq hs;
    if (load_head(&hs, J->q, J->k, J->v, J->N, J->H, J->dk, J->dv, b, h, J->theta, J->pos0)) {
        free_head(&hs);
        return -3;
    }
    for (int n = 0; n < J->N; ++n)
        parallel_row(&hs, J->dk, J->dv, J->gamma[h], n, out_row(J->o, J->N, J->H, J->dv, b, n, h));
    free_head(&hs);
    return 0;
}

/* Selected rows only: out is [B][nrows][H][dv]. */
static int form_parallel_rows(job* J, int b, int h) {
    head_seq hs;
    if (load_head(&hs, J->q, J->k, J->v, J->N, J->H, J->dk, J->dv, b, h, J->theta, J->pos0)) {
        free_head(&hs);
        return -3;
    }
    for (int r = 0; r < J->nrows; ++r) {
        long long n = J->rows[r];
        double* o = J->o + (((size_t)b * J->nrows + r) * J->H + h) * (size_t)J->dv;
        parallel_row(&hs, J->dk, J->dv, J->gamma[h], (int)n, o);
    }
    free_head(&hs);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Parallel form with the score normalizations (blog section 8.5; paper summary, "Retention Score     */
/* Normalization"), each switched on by a flag, applied in the pages' order:                         */
/*   1. QK^T is divided by sqrt(d_k) (the pages' d is the q/k head dimension: the attention scaling); */
/*   2. row n of the decay matrix is divided by the square root of its sum over the sequence so far:   */
/*      D~[n][m] = D[n][m] / sqrt(sum_{i<=n} D[n][i]), 0-indexed;                                      */
/*   3. R = (scaled QK^T) (.) D (or D~); row n is divided by max(|sum_m R[n][m]|, 1).                   */
/* Output o_n = sum_m R~[n][m] v_m. Every factor is a scalar per (token, head).                      */
/* ------------------------------------------------------------------------------------------------ */

#define ORC_NORM_SCALE 1
#define ORC_NORM_DECAY 2
#define ORC_NORM_SCORES 4

static int form_parallel_norm(job* J, int b, int h) {
    head_seq hs;
    const int N = J->N, dk = J->dk, dv = J->dv;
    const double gamma = J->gamma[h];
    double* w = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!w || load_head(&hs, J->q, J->k, J->v, N, J->H, dk, dv, b, h, J->theta, J->pos0)) {
        free(w);
        free_head(&hs);
        return -3;
    }
    for (int n = 0; n < N; ++n) {
        double dsum = 0.0; /* sum_{i<=n} D[n][i] */
        for (int i = 0; i <= n; ++i) dsum += pow(gamma, (double)(n - i));
        double rsum = 0.0;
        for (int m = 0; m <= n; ++m) {
            double qk = dot(hs.Qr + (size_t)n * dk, hs.Kr + (size_t)m * dk, dk);
            if (J->norm & ORC_NORM_SCALE) qk /= sqrt((double)dk);
            double D = pow(gamma, (double)(n - m));
            if (J->norm & ORC_NORM_DECAY) D /= sqrt(dsum);
            w[m] = qk * D;
            rsum += w[m];
        }
        double den = 1.0;
        if (J->norm & ORC_NORM_SCORES) den = fabs(rsum) > 1.0 ? fabs(rsum) : 1.0;
        double* o = out_row(J->o, N, J->H, dv, b, n, h);
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int m = 0; m <= n; ++m) {
            const double* vm = hs.Vh + (size_t)m * dv;
            for (int j = 0; j < dv; ++j) o[j] += (w[m] / den) * vm[j];
        }
    }
    free(w);
    free_head(&hs);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Gradients of the recurrent form, from a zero state, given dO = dL/dO (the adjoint of the scan):      */
/*   forward:  S_n = gamma S_{n-1} + k'_n^T v_n,   dq'_n[i] = sum_j S_n[i][j] dO_n[j];                  */
/*   backward: G_n = gamma G_{n+1} + q'_n^T dO_n,  dk'_n[i] = sum_j G_n[i][j] v_n[j],                    */
/*             dv_n[j] = sum_i k'_n[i] G_n[i][j];                                                       */
/* then the rotation's transpose: (dx_{2i}, dx_{2i+1}) = (c dx'_{2i} + s dx'_{2i+1}, -s dx'_{2i} + c dx'_{2i+1}) */
/* with c, s of the angle (pos0 + n) theta_i, for dq and dk.                                           */
/* ------------------------------------------------------------------------------------------------ */

static void unrotate_row(double* d, int dk, const double* theta, long long p) {
    if (!theta) return;
    for (int i = 0; i < dk / 2; ++i) {
        double phi = (double)p * theta[i];
        double c = cos(phi), s = sin(phi);
        double a = d[2 * i], b = d[2 * i + 1];
        d[2 * i] = c * a + s * b;
        d[2 * i + 1] = -s * a + c * b;
    }
}

static int form_grad(job* J, int b, int h) {
    const int N = J->N, H = J->H, dk = J->dk, dv = J->dv;
    const double g = J->gamma[h];
    head_seq hs;
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* dO = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * dv);
    if (!S || !dO || load_head(&hs, J->q, J->k, J->v, N, H, dk, dv, b, h, J->theta, J->pos0)) {
        free(S);
        free(dO);
        free_head(&hs);
        return -3;
    }
    for (int n = 0; n < N; ++n) gather_plain(J->dout, dO + (size_t)n * dv, N, H, dv, b, n, h);
    for (int n = 0; n < N; ++n) {
        const double* kn = hs.Kr + (size_t)n * dk;
        const double* vn = hs.Vh + (size_t)n * dv;
        const double* don = dO + (size_t)n * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kn[i] * vn[j];
        double* dq = out_row(J->dq, N, H, dk, b, n, h);
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += S[(size_t)i * dv + j] * don[j];
            dq[i] = acc;
        }
        unrotate_row(dq, dk, J->theta, J->pos0 + n);
    }
    memset(S, 0, sizeof(double) * (size_t)dk * dv); /* S now holds G */
    for (int n = N - 1; n >= 0; --n) {
        const double* qn = hs.Qr + (size_t)n * dk;
        const double* kn = hs.Kr + (size_t)n * dk;
        const double* vn = hs.Vh + (size_t)n * dv;
        const double* don = dO + (size_t)n * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + qn[i] * don[j];
        double* dkr = out_row(J->dk_, N, H, dk, b, n, h);
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += S[(size_t)i * dv + j] * vn[j];
            dkr[i] = acc;
        }
        unrotate_row(dkr, dk, J->theta, J->pos0 + n);
        double* dvr = out_row(J->dv_, N, H, dv, b, n, h);
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += kn[i] * S[(size_t)i * dv + j];
            dvr[j] = acc;
        }
    }
    free(S);
    free(dO);
    free_head(&hs);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Recurrent form (blog section 2.1; paper summary Eq. 6): S <- gamma S + k_n^T v_n, then o_n = q_n S.*/
/* ------------------------------------------------------------------------------------------------ */

static int form_recurrent(job* J, int b, int h) {
    const int N = J->N, H = J->H, dk = J->dk, dv = J->dv;
    const double g = J->gamma[h];
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* qr = (double*)malloc(sizeof(double) * dk);
    double* kr = (double*)malloc(sizeof(double) * dk);
    if (!S || !qr || !kr) {
        free(S); free(qr); free(kr);
        return -3;
    }
    size_t soff = ((size_t)b * H + h) * (size_t)dk * dv;
    if (J->s_in) memcpy(S, J->s_in + soff, sizeof(double) * (size_t)dk * dv);
    for (int n = 0; n < N; ++n) {
        gather_rotated(J->q, qr, N, H, dk, b, n, h, J->theta, J->pos0 + n);
        gather_rotated(J->k, kr, N, H, dk, b, n, h, J->theta, J->pos0 + n);
        const double* vn = J->v + (((size_t)b * N + n) * H + h) * (size_t)dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kr[i] * vn[j];
        double* on = out_row(J->o, N, H, dv, b, n, h);
        for (int j = 0; j < dv; ++j) on[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) on[j] += qr[i] * S[(size_t)i * dv + j];
    }
    if (J->s_out) memcpy(J->s_out + soff, S, sizeof(double) * (size_t)dk * dv);
    free(S); free(qr); free(kr);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Chunkwise form (blog section 7.2; paper summary Eq. 7), chunk i = tokens [t0, t0 + L):            */
/*   inner = (Q_c K_c^T (.) D_chunk) V_c,           D_chunk[j][l] = gamma^(j-l), j >= l               */
/*   cross = (Q_c R) (.) xi,                        xi_j   = gamma^(j+1)  (j counted from 0)          */
/*   R    <- gamma^L R + K_c^T (V_c (.) zeta),      zeta_l = gamma^(L-1-l)                            */
/* ------------------------------------------------------------------------------------------------ */

static int form_chunkwise(job* J, int b, int h) {
    const int N = J->N, H = J->H, dk = J->dk, dv = J->dv, C = J->chunk;
    const double g = J->gamma[h];
    head_seq hs;
    double* R = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* A = (double*)malloc(sizeof(double) * (size_t)C * C + 8);    /* Q_c K_c^T (.) D_chunk */
    double* QR = (double*)malloc(sizeof(double) * (size_t)C * dv + 8);  /* Q_c R                 */
    double* Vz = (double*)malloc(sizeof(double) * (size_t)C * dv + 8);  /* V_c (.) zeta          */
    double* U = (double*)malloc(sizeof(double) * (size_t)dk * dv + 8);  /* K_c^T (V_c (.) zeta)  */
    int rc = load_head(&hs, J->q, J->k, J->v, N, H, dk, dv, b, h, J->theta, J->pos0);
    if (rc || !R || !A || !QR || !Vz || !U) {
        free_head(&hs); free(R); free(A); free(QR); free(Vz); free(U);
        return -3;
    }
    size_t soff = ((size_t)b * H + h) * (size_t)dk * dv;
    if (J->s_in) memcpy(R, J->s_in + soff, sizeof(double) * (size_t)dk * dv);

    for (int t0 = 0; t0 < N; t0 += C) {
        const int L = (N - t0 < C) ? (N - t0) : C;
        const double* Qc = hs.Qr + (size_t)t0 * dk;
        const double* Kc = hs.Kr + (size_t)t0 * dk;
        const double* Vc = hs.Vh + (size_t)t0 * dv;

        /* Inner-chunk scores with the causal decay mask D_chunk. */
        for (int j = 0; j < L; ++j)
            for (int l = 0; l < L; ++l)
                A[(size_t)j * C + l] = (l <= j) ? dot(Qc + (size_t)j * dk, Kc + (size_t)l * dk, dk) *
                                                      pow(g, (double)(j - l))
                                                : 0.0;
        /* Cross-chunk read of the carried state, before it is updated: QR = Q_c R. */
        for (int j = 0; j < L; ++j) {
            double* qr = QR + (size_t)j * dv;
            for (int c = 0; c < dv; ++c) qr[c] = 0.0;
            for (int i = 0; i < dk; ++i) {
                const double qi = Qc[(size_t)j * dk + i];
                const double* Ri = R + (size_t)i * dv;
                for (int c = 0; c < dv; ++c) qr[c] += qi * Ri[c];
            }
        }
        /* Output row j = inner_j + xi_j * QR_j, inner = (A (.) D) V_c. */
        for (int j = 0; j < L; ++j) {
            double* oj = out_row(J->o, N, H, dv, b, t0 + j, h);
            for (int c = 0; c < dv; ++c) oj[c] = 0.0;
            for (int l = 0; l < L; ++l) {
                const double a = A[(size_t)j * C + l];
                const double* vl = Vc + (size_t)l * dv;
                for (int c = 0; c < dv; ++c) oj[c] += a * vl[c];
            }
            const double xi = pow(g, (double)(j + 1));
            for (int c = 0; c < dv; ++c) oj[c] += QR[(size_t)j * dv + c] * xi;
        }
        /* State carry: U = K_c^T (V_c (.) zeta), then R <- gamma^L R + U. */
        for (int l = 0; l < L; ++l) {
            const double zeta = pow(g, (double)(L - 1 - l));
            for (int c = 0; c < dv; ++c) Vz[(size_t)l * dv + c] = Vc[(size_t)l * dv + c] * zeta;
        }
        for (size_t e = 0; e < (size_t)dk * dv; ++e) U[e] = 0.0;
        for (int l = 0; l < L; ++l)
            for (int i = 0; i < dk; ++i) {
                const double ki = Kc[(size_t)l * dk + i];
                const double* vz = Vz + (size_t)l * dv;
                double* Ui = U + (size_t)i * dv;
                for (int c = 0; c < dv; ++c) Ui[c] += ki * vz[c];
            }
        const double gL = pow(g, (double)L);
        for (size_t e = 0; e < (size_t)dk * dv; ++e) R[e] = gL * R[e] + U[e];
    }
    if (J->s_out) memcpy(J->s_out + soff, R, sizeof(double) * (size_t)dk * dv);
    free_head(&hs); free(R); free(A); free(QR); free(Vz); free(U);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Score normalizations through a carried state. The pages define them on the parallel form only (blog */
/* section 8.5; paper summary, "Retention Score Normalization"). Reading: each refers to the whole      */
/* sequence from its first token, so row n of a call that starts at absolute position pos0 is row       */
/* p = pos0 + n of the sequence, and                                                                  */
/*   c_p  = (scale ? 1/sqrt(d_k) : 1) * (decay ? 1/sqrt(sum_{i<=p} D[p][i]) : 1),                     */
/*          sum_{i<=p} D[p][i] = sum_{m=0}^{p} gamma^(p-m)                                            */
/*   r_p  = sum_{m<=p} c_p gamma^(p-m) (q'_p . k'_m) = c_p (q'_p . z_p),   z_p = gamma z_{p-1} + k'_p  */
/*   o~_p = c_p o_p / (scores ? max(|r_p|, 1) : 1),   o_p the plain retention output.                 */
/* z (d_k values per (b, h)) is the decayed sum of the rotated keys; z_in is z before the call's first */
/* token (NULL: zero, a fresh sequence).                                                              */
/* ------------------------------------------------------------------------------------------------ */

/* Row p's sum of the decay matrix, sum_{m=0}^{p} gamma^(p-m), written out term by term. */
static double decay_row_sum(double g, long long p) {
    double s = 0.0;
    for (long long m = 0; m <= p; ++m) s += pow(g, (double)(p - m));
    return s;
}

/* The factor c_p / den_p that turns the plain output of row p into the normalized one, given q'_p . z_p. */
static double norm_row_factor(int norm, int dk, double g, long long p, double qz) {
    double c = 1.0;
    if (norm & ORC_NORM_SCALE) c /= sqrt((double)dk);
    if (norm & ORC_NORM_DECAY) c /= sqrt(decay_row_sum(g, p));
    double den = 1.0;
    if (norm & ORC_NORM_SCORES) {
        const double r = c * qz;
        den = fabs(r) > 1.0 ? fabs(r) : 1.0;
    }
    return c / den;
}

/* Recurrent form with the normalizations: S <- gamma S + k'^T v, z <- gamma z + k', o = c (q' S) / den. */
static int form_recurrent_norm(job* J, int b, int h) {
    const int N = J->N, H = J->H, dk = J->dk, dv = J->dv;
    const double g = J->gamma[h];
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* z = (double*)calloc((size_t)dk, sizeof(double));
    double* qr = (double*)malloc(sizeof(double) * dk);
    double* kr = (double*)malloc(sizeof(double) * dk);
    if (!S || !z || !qr || !kr) {
        free(S); free(z); free(qr); free(kr);
        return -3;
    }
    const size_t soff = ((size_t)b * H + h) * (size_t)dk * dv, zoff = ((size_t)b * H + h) * (size_t)dk;
    if (J->s_in) memcpy(S, J->s_in + soff, sizeof(double) * (size_t)dk * dv);
    if (J->z_in) memcpy(z, J->z_in + zoff, sizeof(double) * (size_t)dk);
    for (int n = 0; n < N; ++n) {
        const long long p = J->pos0 + n;
        gather_rotated(J->q, qr, N, H, dk, b, n, h, J->theta, p);
        gather_rotated(J->k, kr, N, H, dk, b, n, h, J->theta, p);
        const double* vn = J->v + (((size_t)b * N + n) * H + h) * (size_t)dv;
        for (int i = 0; i < dk; ++i) {
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kr[i] * vn[j];
            z[i] = g * z[i] + kr[i];
        }
        double* on = out_row(J->o, N, H, dv, b, n, h);
        for (int j = 0; j < dv; ++j) on[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) on[j] += qr[i] * S[(size_t)i * dv + j];
        const double f = norm_row_factor(J->norm, dk, g, p, dot(qr, z, dk));
        for (int j = 0; j < dv; ++j) on[j] *= f;
    }
    if (J->s_out) memcpy(J->s_out + soff, S, sizeof(double) * (size_t)dk * dv);
    if (J->z_out) memcpy(J->z_out + zoff, z, sizeof(double) * (size_t)dk);
    free(S); free(z); free(qr); free(kr);
    return 0;
}

/* Chunkwise form with the normalizations: the plain chunkwise outputs and state (form_chunkwise), and the row
 * sums q'_j . z_j of each chunk [t0, t0 + L) computed the chunkwise way, as the outputs are:
 *   q'_j . z_j = sum_{l<=j} gamma^(j-l) (q'_j . k'_l) + gamma^(j+1) (q'_j . z),   z <- gamma^L z + sum_l zeta_l k'_l
 * with z the decayed key sum entering the chunk; each output row is then scaled by its factor. */
static int form_chunkwise_norm(job* J, int b, int h) {
    int rc = form_chunkwise(J, b, h);
    if (rc) return rc;
    const int N = J->N, H = J->H, dk = J->dk, dv = J->dv, C = J->chunk;
    const double g = J->gamma[h];
    head_seq hs;
    double* z = (double*)calloc((size_t)dk, sizeof(double));
    double* rs = (double*)malloc(sizeof(double) * (size_t)C + 8);
    rc = load_head(&hs, J->q, J->k, J->v, N, H, dk, dv, b, h, J->theta, J->pos0);
    if (rc || !z || !rs) {
        free_head(&hs); free(z); free(rs);
        return -3;
    }
    const size_t zoff = ((size_t)b * H + h) * (size_t)dk;
    if (J->z_in) memcpy(z, J->z_in + zoff, sizeof(double) * (size_t)dk);
    for (int t0 = 0; t0 < N; t0 += C) {
        const int L = (N - t0 < C) ? (N - t0) : C;
        const double* Qc = hs.Qr + (size_t)t0 * dk;
        const double* Kc = hs.Kr + (size_t)t0 * dk;
        for (int j = 0; j < L; ++j) {
            double inner = 0.0;
            for (int l = 0; l <= j; ++l) inner += pow(g, (double)(j - l)) * dot(Qc + (size_t)j * dk, Kc + (size_t)l * dk, dk);
            rs[j] = inner + pow(g, (double)(j + 1)) * dot(Qc + (size_t)j * dk, z, dk);
        }
        for (int i = 0; i < dk; ++i) {
            double u = 0.0;
            for (int l = 0; l < L; ++l) u += pow(g, (double)(L - 1 - l)) * Kc[(size_t)l * dk + i];
            z[i] = pow(g, (double)L) * z[i] + u;
        }
        for (int j = 0; j < L; ++j) {
            const double f = norm_row_factor(J->norm, dk, g, J->pos0 + t0 + j, rs[j]);
            double* oj = out_row(J->o, N, H, dv, b, t0 + j, h);
            for (int c = 0; c < dv; ++c) oj[c] *= f;
        }
    }
    if (J->z_out) memcpy(J->z_out + zoff, z, sizeof(double) * (size_t)dk);
    free_head(&hs); free(z); free(rs);
    return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* Exported entry points. Return 0 on success, -1 bad arguments, -2 thread error, -3 out of memory. */
/* ------------------------------------------------------------------------------------------------ */

int orc_parallel(const double* q, const double* k, const double* v, double* o, int B, int N, int H, int dk,
                 int dv, const double* gamma, const double* theta, long long pos0, int nthreads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !o) return -1;
    job J = {0};
    J.q = q; J.k = k; J.v = v; J.o = o; J.gamma = gamma; J.theta = theta;
    J.B = B; J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.pos0 = pos0; J.form = 0; J.nthreads = nthreads;
    return run(J);
}

/* The parallel form with the score normalizations selected by norm (ORC_NORM_* flags). */
int orc_parallel_normalized(const double* q, const double* k, const double* v, double* o, int B, int N, int H,
                            int dk, int dv, const double* gamma, const double* theta, long long pos0, int norm,
                            int threads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !o || norm < 0 || norm > 7) return -1;
    job J;
    memset(&J, 0, sizeof(J));
    J.q = q;
    J.k = k;
    J.v = v;
    J.o = o;
    J.gamma = gamma;
    J.theta = theta;
    J.B = B;
    J.N = N;
    J.H = H;
    J.dk = dk;
    J.dv = dv;
    J.pos0 = pos0;
    J.form = 4;
    J.norm = norm;
    J.nthreads = threads;
    return run(J);
}

/* Multi-scale retention epilogue (blog sections 8.4 and 9.1; paper summary, "Gating mechanism"):
 *   y = swish(g) (.) GroupNorm_h(o).
 * o, g, y: [rows][H][dv] (rows = B*N tokens, or B for one decode step). GroupNorm has one group per head:
 * each (row, head) vector of dv values is standardized by its own mean and biased variance,
 * (x - mean) / sqrt(var + eps), then multiplied by weight[h*dv + c] and shifted by bias[h*dv + c] (either
 * NULL: 1 and 0). swish(x) = x sigmoid(x). g NULL: no gate. y may equal o. */
int orc_msr_epilogue(const double* o, const double* g, const double* weight, const double* bias, double* y,
                     long long rows, int H, int dv, double eps) {
    if (!o || !y || rows < 0 || H <= 0 || dv <= 0 || !(eps >= 0.0)) return -1;
    for (long long r = 0; r < rows; ++r)
        for (int h = 0; h < H; ++h) {
            const size_t base = ((size_t)r * H + h) * (size_t)dv;
            double mean = 0.0, var = 0.0;
            for (int c = 0; c < dv; ++c) mean += o[base + c];
            mean /= dv;
            for (int c = 0; c < dv; ++c) var += (o[base + c] - mean) * (o[base + c] - mean);
            var /= dv;
            const double inv = 1.0 / sqrt(var + eps);
            for (int c = 0; c < dv; ++c) {
                double z = (o[base + c] - mean) * inv;
                const size_t ch = (size_t)h * dv + c;
                if (weight) z *= weight[ch];
                if (bias) z += bias[ch];
                if (g) z *= g[base + c] / (1.0 + exp(-g[base + c]));
                y[base + c] = z;
            }
        }
    return 0;
}

/* Gradients of sum(dout (.) O) with respect to q, k and v, O the retention output from a zero state. */
int orc_grad(const double* q, const double* k, const double* v, const double* dout, double* dq, double* dk_,
             double* dv_, int B, int N, int H, int dk, int dv, const double* gamma, const double* theta,
             long long pos0, int threads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !dout || !dq || !dk_ || !dv_) return -1;
    job J;
    memset(&J, 0, sizeof(J));
    J.q = q;
    J.k = k;
    J.v = v;
    J.dout = dout;
    J.dq = dq;
    J.dk_ = dk_;
    J.dv_ = dv_;
    J.gamma = gamma;
    J.theta = theta;
    J.B = B;
    J.N = N;
    J.H = H;
    J.dk = dk;
    J.dv = dv;
    J.pos0 = pos0;
    J.form = 5;
    J.nthreads = threads;
    return run(J);
}

int orc_parallel_rows(const double* q, const double* k, const double* v, int B, int N, int H, int dk, int dv,
                      const double* gamma, const double* theta, long long pos0, const long long* rows,
                      int nrows, double* o_rows, int nthreads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !o_rows || !rows || nrows <= 0)
        return -1;
    for (int r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N) return -1;
    job J = {0};
    J.q = q; J.k = k; J.v = v; J.o = o_rows; J.gamma = gamma; J.theta = theta; J.rows = rows;
    J.nrows = nrows;
    J.B = B; J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.pos0 = pos0; J.form = 3; J.nthreads = nthreads;
    return run(J);
}

int orc_recurrent(const double* q, const double* k, const double* v, double* o, int B, int N, int H, int dk,
                  int dv, const double* gamma, const double* theta, long long pos0, const double* s_in,
                  double* s_out, int nthreads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !o) return -1;
    job J = {0};
    J.q = q; J.k = k; J.v = v; J.o = o; J.gamma = gamma; J.theta = theta; J.s_in = s_in; J.s_out = s_out;
    J.B = B; J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.pos0 = pos0; J.form = 1; J.nthreads = nthreads;
    return run(J);
}

int orc_chunkwise(const double* q, const double* k, const double* v, double* o, int B, int N, int H, int dk,
                  int dv, const double* gamma, const double* theta, long long pos0, int chunk,
                  const double* s_in, double* s_out, int nthreads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !o || chunk <= 0) return -1;
    job J = {0};
    J.q = q; J.k = k; J.v = v; J.o = o; J.gamma = gamma; J.theta = theta; J.s_in = s_in; J.s_out = s_out;
    J.B = B; J.N = N; J.H = H; J.dk = dk; J.dv = dv; J.pos0 = pos0; J.chunk = chunk; J.form = 2;
    J.nthreads = nthreads;
    return run(J);
}

/* The recurrent (chunk <= 0) or chunkwise (chunk > 0) form with the score normalizations selected by norm
 * (ORC_NORM_* flags), carrying the state S and the decayed key sum z ([B][H][dk]); z_in NULL means zero. */
int orc_normalized(const double* q, const double* k, const double* v, double* o, int B, int N, int H, int dk,
                   int dv, const double* gamma, const double* theta, long long pos0, int chunk, int norm,
                   const double* s_in, double* s_out, const double* z_in, double* z_out, int nthreads) {
    if (check_args(B, N, H, dk, dv, gamma, theta) || !q || !k || !v || !o || norm < 0 || norm > 7 || pos0 < 0)
        return -1;
    job J;
    memset(&J, 0, sizeof(J));
    J.q = q;
    J.k = k;
    J.v = v;
    J.o = o;
    J.gamma = gamma;
    J.theta = theta;
    J.s_in = s_in;
    J.s_out = s_out;
    J.z_in = z_in;
    J.z_out = z_out;
    J.B = B;
    J.N = N;
    J.H = H;
    J.dk = dk;
    J.dv = dv;
    J.pos0 = pos0;
    J.chunk = chunk;
    J.norm = norm;
    J.form = chunk > 0 ? 7 : 6;
    J.nthreads = nthreads;
    return run(J);
}
