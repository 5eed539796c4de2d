/*
 * jscan_oracle.c - plain, slow, fp64 CPU oracle for the Mamba-1 (S6) selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this
 * file: only the test suite, the smoke check and the CPU-baseline leg of the bench use it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes.  The S6 recurrence of the Jamba notes page ("Jamba: A Hybrid
 * Transformer-Mamba Language Model", section "Mamba layer", the S6 equation) and of the
 * lesson page ("Jamba - Hybrid SSM-Transformer", section "SSM on one page"):
 *
 *     h_t = Abar_t * h_{t-1} + Bbar_t x_t,          y_t = C_t h_t
 *
 * with input-dependent Delta_t, B_t, C_t (notes page, same section) and a real diagonal A
 * (lesson page, section "Mamba-3", item 2).  The discretisation is
 *
 *     Abar_t = exp(Delta_t * A),                    Bbar_t x_t = Delta_t * B_t * x_t
 *
 * Because A is diagonal every (batch b, channel d, state n) is an independent scalar
 * recurrence, and y_t[d] is the dot product of C_t with the state vector h_t[d, :]
 * taken AFTER the update of step t.
 *
 * Layouts (row-major, last index fastest):
 *     x, delta, y : [batch][L][D]          A      : [D][N]
 *     B, C        : [batch][L][N]          h0, h  : [batch][D][N]
 *
 * Every value is a double.  The caller widens bf16 / fp32 inputs exactly to double first.
 * The time loop is strictly sequential; only independent (b, d) chains are spread over
 * threads, which does not change a single rounding.
 */
#include <complex.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *x, *delta, *A, *B, *C, *h0;
    double *y, *h_final;
    int64_t batch, L, D, N, chunk;
    int cplx;                     /* complex-valued state (see scan_chain_complex) */
    int trap;                     /* exponential-trapezoidal rule (see scan_chain_trapezoid) */
    const double *lam;            /* trapezoid weights [batch][L][D] */
    const double *x_prev, *B_prev; /* token before the first: [batch][D], [batch][N]; NULL = none */
    int64_t R;                    /* MIMO rank (see scan_chain_mimo); 0 = single input and output */
    int64_t item_begin, item_end; /* items are (b, d) pairs, item = b * D + d */
} scan_job;

/* One (b, d) chain over all L tokens: the recurrence written out term by term. */
static void scan_chain_sequential(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N;
    double *h = (double *)malloc((size_t)N * sizeof(double));
    for (int64_t n = 0; n < N; ++n)
        h[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const double delta_t = j->delta[(b * L + t) * D + d];
        const double x_t = j->x[(b * L + t) * D + d];
        const double *B_t = j->B + (b * L + t) * N;
        const double *C_t = j->C + (b * L + t) * N;
        double y_t = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double Abar = exp(delta_t * j->A[d * N + n]);     /* Abar_t = exp(Delta_t A)   */
            const double Bbar_x = delta_t * B_t[n] * x_t;           /* Bbar_t x_t = Delta_t B_t x_t */
            h[n] = Abar * h[n] + Bbar_x;                            /* h_t = Abar_t h_{t-1} + Bbar_t x_t */
            y_t += C_t[n] * h[n];                                   /* y_t = C_t h_t             */
        }
        j->y[(b * L + t) * D + d] = y_t;
    }
    if (j->h_final)
        for (int64_t n = 0; n < N; ++n)
            j->h_final[(b * D + d) * N + n] = h[n];
    free(h);
}

/*
 * The same chain evaluated chunk by chunk with the associative combine of the linear
 * recurrence: a chunk of tokens acts on an incoming state as h -> P * h + q, where
 * P = prod(Abar) over the chunk and q is the chunk's own scan started from zero;
 * composing two such maps gives (P1, q1) then (P2, q2) = (P1 P2, P2 q1 + q2).
 * Inside a chunk, h_t = P_{<=t} h_in + q_t.  Used only to pin that chunked evaluation
 * equals the sequential one (the basis of time-parallel and sequence-split scans).
 */
static void scan_chain_chunked(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N, K = j->chunk;
    double *h_in = (double *)malloc((size_t)N * sizeof(double));
    double *P = (double *)malloc((size_t)N * sizeof(double));
    double *q = (double *)malloc((size_t)N * sizeof(double));
    for (int64_t n = 0; n < N; ++n)
        h_in[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;

    for (int64_t t0 = 0; t0 < L; t0 += K) {
        const int64_t t1 = (t0 + K < L) ? t0 + K : L;
        for (int64_t n = 0; n < N; ++n) {
            P[n] = 1.0;
            q[n] = 0.0;
        }
        for (int64_t t = t0; t < t1; ++t) {
            const double delta_t = j->delta[(b * L + t) * D + d];
            const double x_t = j->x[(b * L + t) * D + d];
            const double *B_t = j->B + (b * L + t) * N;
            const double *C_t = j->C + (b * L + t) * N;
            double y_t = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double Abar = exp(delta_t * j->A[d * N + n]);
                P[n] = P[n] * Abar;                              /* product of Abar inside the chunk */
                q[n] = Abar * q[n] + delta_t * B_t[n] * x_t;     /* chunk-local scan from zero        */
                y_t += C_t[n] * (P[n] * h_in[n] + q[n]);         /* state = P h_in + q                */
            }
            j->y[(b * L + t) * D + d] = y_t;
        }
        for (int64_t n = 0; n < N; ++n)
            h_in[n] = P[n] * h_in[n] + q[n];                     /* carry the state into the next chunk */
    }
    if (j->h_final)
        for (int64_t n = 0; n < N; ++n)
            j->h_final[(b * D + d) * N + n] = h_in[n];
    free(h_in);
    free(P);
    free(q);
}

/*
 * Complex-valued state: the Mamba-3 change named on the lesson page ("Jamba - Hybrid
 * SSM-Transformer", section "Mamba-3", item 2), where the state matrix becomes complex again
 * and so multiplies the state by a data-dependent rotation.  The N real components of a
 * channel's state are read as N/2 complex states, h[k] = h[2k] + i h[2k+1].  A holds each
 * complex diagonal entry as (A[2k], A[2k+1]) = (real part, imaginary part), and B and C pair
 * up the same way.  The S6 equation then reads, in complex arithmetic,
 *     Abar_t = exp(Delta_t a_k),  a_k = A[2k] + i A[2k+1]
 *     h_t[k] = Abar_t h_{t-1}[k] + Delta_t x_t b_k,  b_k = B_t[2k] + i B_t[2k+1]
 *     y_t    = sum_k Re(conj(c_k) h_t[k]),  c_k = C_t[2k] + i C_t[2k+1]
 * and the output is the same dot product of C_t with the N real components as in the real
 * scan.  With every imaginary part of A zero it is the real scan with A[2k+1] = A[2k].
 */
static void scan_chain_complex(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N, K = N / 2;
    double complex *h = (double complex *)malloc((size_t)K * sizeof(double complex));
    for (int64_t k = 0; k < K; ++k)
        h[k] = j->h0 ? j->h0[(b * D + d) * N + 2 * k] + I * j->h0[(b * D + d) * N + 2 * k + 1] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const double delta_t = j->delta[(b * L + t) * D + d];
        const double x_t = j->x[(b * L + t) * D + d];
        const double *B_t = j->B + (b * L + t) * N;
        const double *C_t = j->C + (b * L + t) * N;
        double y_t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double complex a = j->A[d * N + 2 * k] + I * j->A[d * N + 2 * k + 1];
            const double complex Abar = cexp(delta_t * a);
            const double complex bk = B_t[2 * k] + I * B_t[2 * k + 1];
            const double complex ck = C_t[2 * k] + I * C_t[2 * k + 1];
            h[k] = Abar * h[k] + delta_t * x_t * bk;
            y_t += creal(conj(ck) * h[k]);
        }
        j->y[(b * L + t) * D + d] = y_t;
    }
    if (j->h_final)
        for (int64_t k = 0; k < K; ++k) {
            j->h_final[(b * D + d) * N + 2 * k] = creal(h[k]);
            j->h_final[(b * D + d) * N + 2 * k + 1] = cimag(h[k]);
        }
    free(h);
}

/*
 * Exponential-trapezoidal discretisation: the first Mamba-3 change named on the lesson page
 * ("Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 1), which replaces the Euler
 * rule by a recurrence that mixes the state input of neighbouring tokens inside the scan.
 * Written out from the continuous system h' = A h + B(s) x(s): over one step of length
 * Delta_t the state decays by Abar_t = exp(Delta_t A) and takes in the integral of
 * exp((Delta_t - u) A) B x over the step.  The Euler rule keeps only the step's right end
 * point (Delta_t B_t x_t).  A two-point rule weights the right end by lambda_t and the left
 * end, which has decayed over the whole step, by 1 - lambda_t:
 *
 *     h_t = Abar_t h_{t-1} + (1 - lambda_t) Delta_t Abar_t B_{t-1} x_{t-1} + lambda_t Delta_t B_t x_t
 *
 * lambda_t = 1 is the Euler rule; lambda_t = 1/2 is the trapezoid rule, second-order accurate
 * in Delta where the Euler rule is first-order.  The token before the first one is
 * (x_prev, B_prev) when given (a resumed sequence), else there is none and its term is zero.
 * y_t = C_t h_t as before.
 */
static void scan_chain_trapezoid(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N;
    double *h = (double *)malloc((size_t)N * sizeof(double));
    double *u_prev = (double *)malloc((size_t)N * sizeof(double));   /* B_{t-1} x_{t-1} */
    for (int64_t n = 0; n < N; ++n) {
        h[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;
        u_prev[n] = j->x_prev ? j->B_prev[b * N + n] * j->x_prev[b * D + d] : 0.0;
    }
    for (int64_t t = 0; t < L; ++t) {
        const double delta_t = j->delta[(b * L + t) * D + d];
        const double lam_t = j->lam[(b * L + t) * D + d];
        const double x_t = j->x[(b * L + t) * D + d];
        const double *B_t = j->B + (b * L + t) * N;
        const double *C_t = j->C + (b * L + t) * N;
        double y_t = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double Abar = exp(delta_t * j->A[d * N + n]);
            const double u_t = B_t[n] * x_t;
            h[n] = Abar * h[n] + (1.0 - lam_t) * delta_t * Abar * u_prev[n] + lam_t * delta_t * u_t;
            u_prev[n] = u_t;
            y_t += C_t[n] * h[n];
        }
        j->y[(b * L + t) * D + d] = y_t;
    }
    if (j->h_final)
        for (int64_t n = 0; n < N; ++n)
            j->h_final[(b * D + d) * N + n] = h[n];
    free(h);
    free(u_prev);
}

/* The same rule with the complex-valued state of scan_chain_complex. */
static void scan_chain_trapezoid_complex(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N, K = N / 2;
    double complex *h = (double complex *)malloc((size_t)K * sizeof(double complex));
    double complex *u_prev = (double complex *)malloc((size_t)K * sizeof(double complex));
    for (int64_t k = 0; k < K; ++k) {
        h[k] = j->h0 ? j->h0[(b * D + d) * N + 2 * k] + I * j->h0[(b * D + d) * N + 2 * k + 1] : 0.0;
        u_prev[k] = j->x_prev
                        ? (j->B_prev[b * N + 2 * k] + I * j->B_prev[b * N + 2 * k + 1]) * j->x_prev[b * D + d]
                        : 0.0;
    }
    for (int64_t t = 0; t < L; ++t) {
        const double delta_t = j->delta[(b * L + t) * D + d];
        const double lam_t = j->lam[(b * L + t) * D + d];
        const double x_t = j->x[(b * L + t) * D + d];
        const double *B_t = j->B + (b * L + t) * N;
        const double *C_t = j->C + (b * L + t) * N;
        double y_t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double complex a = j->A[d * N + 2 * k] + I * j->A[d * N + 2 * k + 1];
            const double complex Abar = cexp(delta_t * a);
            const double complex u_t = (B_t[2 * k] + I * B_t[2 * k + 1]) * x_t;
            const double complex ck = C_t[2 * k] + I * C_t[2 * k + 1];
            h[k] = Abar * h[k] + (1.0 - lam_t) * delta_t * Abar * u_prev[k] + lam_t * delta_t * u_t;
            u_prev[k] = u_t;
            y_t += creal(conj(ck) * h[k]);
        }
        j->y[(b * L + t) * D + d] = y_t;
    }
    if (j->h_final)
        for (int64_t k = 0; k < K; ++k) {
            j->h_final[(b * D + d) * N + 2 * k] = creal(h[k]);
            j->h_final[(b * D + d) * N + 2 * k + 1] = cimag(h[k]);
        }
    free(h);
    free(u_prev);
}

/*
 * Multi-input, multi-output (MIMO) scan: the third Mamba-3 change named on the lesson page
 * ("Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 3), where the per-channel scalar
 * input and output projections become matrix-valued.  Each channel d takes R inputs
 * x_t[d][r] and gives R outputs y_t[d][r]; B_t and C_t are N x R matrices shared by all
 * channels.  The state keeps its size; its input is a rank-R sum instead of one product:
 *
 *     h_t[d][n] = Abar_t[d][n] h_{t-1}[d][n] + Delta_t[d] * sum_r B_t[n][r] x_t[d][r]
 *     y_t[d][r] = sum_n C_t[n][r] h_t[d][n]
 *
 * R = 1 is the single-input scan.  Layouts: x, y [batch][L][D][R]; B, C [batch][L][N][R].
 * With cplx set the state is complex as in scan_chain_complex: pairs (2k, 2k+1) of states,
 * of A's entries and of B's and C's rows (for each r) are complex numbers, and
 * y_t[d][r] = sum_k Re(conj(c_k,r) h_t[k]).
 */
/* The rank-R input of state n: sum_r B[n][r] x[r]. */
static double mimo_u(const double *B, const double *x, int64_t n, int64_t R)
{
    double u = 0.0;
    for (int64_t r = 0; r < R; ++r)
        u += B[n * R + r] * x[r];
    return u;
}

/*
 * With the exponential-trapezoidal rule as well (j->trap), the input term of scan_chain_trapezoid
 * with the rank-R input u in place of B x:
 *     h_t = Abar_t h_{t-1} + (1 - lambda_t) Delta_t Abar_t u_{t-1} + lambda_t Delta_t u_t
 * the token before the first being (x_prev [batch][D][R], B_prev [batch][N][R]) or none.
 */
static void scan_chain_mimo(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N, R = j->R;
    double *h = (double *)malloc((size_t)N * sizeof(double));
    double *u_prev = (double *)malloc((size_t)N * sizeof(double));
    for (int64_t n = 0; n < N; ++n) {
        h[n] = j->h0 ? j->h0[(b * D + d) * N + n] : 0.0;
        u_prev[n] = (j->trap && j->x_prev) ? mimo_u(j->B_prev + b * N * R, j->x_prev + (b * D + d) * R, n, R) : 0.0;
    }
    for (int64_t t = 0; t < L; ++t) {
        const double delta_t = j->delta[(b * L + t) * D + d];
        const double lam_t = j->trap ? j->lam[(b * L + t) * D + d] : 1.0;
        const double *x_t = j->x + ((b * L + t) * D + d) * R;
        const double *B_t = j->B + (b * L + t) * N * R;
        const double *C_t = j->C + (b * L + t) * N * R;
        double *y_t = j->y + ((b * L + t) * D + d) * R;
        for (int64_t n = 0; n < N; ++n) {
            const double Abar = exp(delta_t * j->A[d * N + n]);
            const double u = mimo_u(B_t, x_t, n, R);
            if (j->trap)
                h[n] = Abar * h[n] + (1.0 - lam_t) * delta_t * Abar * u_prev[n] + lam_t * delta_t * u;
            else
                h[n] = Abar * h[n] + delta_t * u;
            u_prev[n] = u;
        }
        for (int64_t r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n)
                acc += C_t[n * R + r] * h[n];
            y_t[r] = acc;
        }
    }
    if (j->h_final)
        for (int64_t n = 0; n < N; ++n)
            j->h_final[(b * D + d) * N + n] = h[n];
    free(h);
    free(u_prev);
}

/* The rank-R complex input of complex state k: sum_r (B[2k][r] + i B[2k+1][r]) x[r]. */
static double complex mimo_u_complex(const double *B, const double *x, int64_t k, int64_t R)
{
    double complex u = 0.0;
    for (int64_t r = 0; r < R; ++r)
        u += (B[2 * k * R + r] + I * B[(2 * k + 1) * R + r]) * x[r];
    return u;
}

static void scan_chain_mimo_complex(const scan_job *j, int64_t b, int64_t d)
{
    const int64_t L = j->L, D = j->D, N = j->N, R = j->R, K = N / 2;
    double complex *h = (double complex *)malloc((size_t)K * sizeof(double complex));
    double complex *u_prev = (double complex *)malloc((size_t)K * sizeof(double complex));
    for (int64_t k = 0; k < K; ++k) {
        h[k] = j->h0 ? j->h0[(b * D + d) * N + 2 * k] + I * j->h0[(b * D + d) * N + 2 * k + 1] : 0.0;
        u_prev[k] = (j->trap && j->x_prev)
                        ? mimo_u_complex(j->B_prev + b * N * R, j->x_prev + (b * D + d) * R, k, R)
                        : 0.0;
    }
    for (int64_t t = 0; t < L; ++t) {
        const double delta_t = j->delta[(b * L + t) * D + d];
        const double lam_t = j->trap ? j->lam[(b * L + t) * D + d] : 1.0;
        const double *x_t = j->x + ((b * L + t) * D + d) * R;
        const double *B_t = j->B + (b * L + t) * N * R;
        const double *C_t = j->C + (b * L + t) * N * R;
        double *y_t = j->y + ((b * L + t) * D + d) * R;
        for (int64_t k = 0; k < K; ++k) {
            const double complex a = j->A[d * N + 2 * k] + I * j->A[d * N + 2 * k + 1];
            const double complex Abar = cexp(delta_t * a);
            const double complex u = mimo_u_complex(B_t, x_t, k, R);
            if (j->trap)
                h[k] = Abar * h[k] + (1.0 - lam_t) * delta_t * Abar * u_prev[k] + lam_t * delta_t * u;
            else
                h[k] = Abar * h[k] + delta_t * u;
            u_prev[k] = u;
        }
        for (int64_t r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += creal(conj(C_t[2 * k * R + r] + I * C_t[(2 * k + 1) * R + r]) * h[k]);
            y_t[r] = acc;
        }
    }
    if (j->h_final)
        for (int64_t k = 0; k < K; ++k) {
            j->h_final[(b * D + d) * N + 2 * k] = creal(h[k]);
            j->h_final[(b * D + d) * N + 2 * k + 1] = cimag(h[k]);
        }
    free(h);
    free(u_prev);
}

static void *scan_worker(void *arg)
{
    const scan_job *j = (const scan_job *)arg;
    for (int64_t item = j->item_begin; item < j->item_end; ++item) {
        const int64_t b = item / j->D, d = item % j->D;
        if (j->R > 0 && j->cplx)
            scan_chain_mimo_complex(j, b, d);
        else if (j->R > 0)
            scan_chain_mimo(j, b, d);
        else if (j->trap && j->cplx)
            scan_chain_trapezoid_complex(j, b, d);
        else if (j->trap)
            scan_chain_trapezoid(j, b, d);
        else if (j->cplx)
            scan_chain_complex(j, b, d);
        else if (j->chunk > 0)
            scan_chain_chunked(j, b, d);
        else
            scan_chain_sequential(j, b, d);
    }
    return NULL;
}

static int run_scan(scan_job base, int nthreads)
{
    const int64_t items = base.batch * base.D;
    if (items <= 0 || base.L <= 0)
        return 0;
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if (nthreads > items)
        nthreads = (int)items;
    pthread_t *tid = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    scan_job *jobs = (scan_job *)malloc((size_t)nthreads * sizeof(scan_job));
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = base;
        jobs[i].item_begin = items * i / nthreads;
        jobs[i].item_end = items * (i + 1) / nthreads;
        if (pthread_create(&tid[i], NULL, scan_worker, &jobs[i]) != 0) {
            scan_worker(&jobs[i]); /* fall back to running this share inline */
            continue;
        }
        tid[started] = tid[i];
        ++started;
    }
    for (int i = 0; i < started; ++i)
        pthread_join(tid[i], NULL);
    free(tid);
    free(jobs);
    return rc;
}

/* Prefill: y for every token and the state after the last token.  h0 may be NULL (zero state). */
int oracle_prefill_f64(const double *x, const double *delta, const double *A, const double *B,
                       const double *C, const double *h0, double *y, double *h_final,
                       int64_t batch, int64_t L, int64_t D, int64_t N, int nthreads)
{
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x; j.delta = delta; j.A = A; j.B = B; j.C = C; j.h0 = h0;
    j.y = y; j.h_final = h_final;
    j.batch = batch; j.L = L; j.D = D; j.N = N; j.chunk = 0;
    return run_scan(j, nthreads);
}

/* Prefill evaluated chunk by chunk (chunk >= 1 tokens) through the associative combine. */
int oracle_prefill_chunked_f64(const double *x, const double *delta, const double *A,
                               const double *B, const double *C, const double *h0, double *y,
                               double *h_final, int64_t batch, int64_t L, int64_t D, int64_t N,
                               int64_t chunk, int nthreads)
{
    if (chunk < 1)
        return -1;
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x; j.delta = delta; j.A = A; j.B = B; j.C = C; j.h0 = h0;
    j.y = y; j.h_final = h_final;
    j.batch = batch; j.L = L; j.D = D; j.N = N; j.chunk = chunk;
    return run_scan(j, nthreads);
}

/*
 * One decode step (constant memory: only h_{t-1} and the current token are needed, lesson
 * page, "SSM on one page").  h is [batch][D][N] and is updated in place; x_t, delta_t and
 * y_t are [batch][D]; B_t and C_t are [batch][N].
 */
int oracle_step_f64(double *h, const double *x_t, const double *delta_t, const double *A,
                    const double *B_t, const double *C_t, double *y_t,
                    int64_t batch, int64_t D, int64_t N)
{
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            const double dl = delta_t[b * D + d], xv = x_t[b * D + d];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double *hn = &h[(b * D + d) * N + n];
                const double Abar = exp(dl * A[d * N + n]);
                *hn = Abar * *hn + dl * B_t[b * N + n] * xv;
                acc += C_t[b * N + n] * *hn;
            }
            y_t[b * D + d] = acc;
        }
    }
    return 0;
}

/* Prefill with the complex-valued state (scan_chain_complex); N must be even. */
int oracle_prefill_complex_f64(const double *x, const double *delta, const double *A, const double *B,
                               const double *C, const double *h0, double *y, double *h_final,
                               int64_t batch, int64_t L, int64_t D, int64_t N, int nthreads)
{
    if (N % 2 != 0)
        return -1;
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x; j.delta = delta; j.A = A; j.B = B; j.C = C; j.h0 = h0;
    j.y = y; j.h_final = h_final;
    j.batch = batch; j.L = L; j.D = D; j.N = N; j.chunk = 0; j.cplx = 1;
    return run_scan(j, nthreads);
}

/* One decode step with the complex-valued state; h [batch][D][N] is updated in place. */
int oracle_step_complex_f64(double *h, const double *x_t, const double *delta_t, const double *A,
                            const double *B_t, const double *C_t, double *y_t,
                            int64_t batch, int64_t D, int64_t N)
{
    if (N % 2 != 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            const double dl = delta_t[b * D + d], xv = x_t[b * D + d];
            double acc = 0.0;
            for (int64_t k = 0; k < N / 2; ++k) {
                double *hk = &h[(b * D + d) * N + 2 * k];
                const double complex a = A[d * N + 2 * k] + I * A[d * N + 2 * k + 1];
                const double complex bk = B_t[b * N + 2 * k] + I * B_t[b * N + 2 * k + 1];
                const double complex ck = C_t[b * N + 2 * k] + I * C_t[b * N + 2 * k + 1];
                const double complex hn = cexp(dl * a) * (hk[0] + I * hk[1]) + dl * xv * bk;
                hk[0] = creal(hn);
                hk[1] = cimag(hn);
                acc += creal(conj(ck) * hn);
            }
            y_t[b * D + d] = acc;
        }
    }
    return 0;
}

/*
 * Prefill with the exponential-trapezoidal rule (scan_chain_trapezoid, or its complex form
 * when cplx is set; N must then be even).  lam is [batch][L][D]; x_prev [batch][D] and
 * B_prev [batch][N] are the token before the first one, both NULL when there is none.
 */
int oracle_prefill_trapezoid_f64(const double *x, const double *delta, const double *lam, const double *A,
                                 const double *B, const double *C, const double *h0, const double *x_prev,
                                 const double *B_prev, double *y, double *h_final, int64_t batch, int64_t L,
                                 int64_t D, int64_t N, int cplx, int nthreads)
{
    if ((cplx && N % 2 != 0) || ((x_prev == NULL) != (B_prev == NULL)))
        return -1;
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x; j.delta = delta; j.A = A; j.B = B; j.C = C; j.h0 = h0;
    j.y = y; j.h_final = h_final;
    j.batch = batch; j.L = L; j.D = D; j.N = N; j.chunk = 0; j.cplx = cplx;
    j.trap = 1; j.lam = lam; j.x_prev = x_prev; j.B_prev = B_prev;
    return run_scan(j, nthreads);
}

/*
 * One decode step with the exponential-trapezoidal rule: the previous token's x_prev [batch][D]
 * and B_prev [batch][N] enter as the step's left end point.  h [batch][D][N] is updated in place.
 */
int oracle_step_trapezoid_f64(double *h, const double *x_prev, const double *B_prev, const double *x_t,
                              const double *delta_t, const double *lam_t, const double *A, const double *B_t,
                              const double *C_t, double *y_t, int64_t batch, int64_t D, int64_t N, int cplx)
{
    if (cplx && N % 2 != 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            const double dl = delta_t[b * D + d], lm = lam_t[b * D + d];
            const double xv = x_t[b * D + d], xp = x_prev[b * D + d];
            double acc = 0.0;
            if (cplx) {
                for (int64_t k = 0; k < N / 2; ++k) {
                    double *hk = &h[(b * D + d) * N + 2 * k];
                    const double complex a = A[d * N + 2 * k] + I * A[d * N + 2 * k + 1];
                    const double complex Abar = cexp(dl * a);
                    const double complex up = (B_prev[b * N + 2 * k] + I * B_prev[b * N + 2 * k + 1]) * xp;
                    const double complex ut = (B_t[b * N + 2 * k] + I * B_t[b * N + 2 * k + 1]) * xv;
                    const double complex ck = C_t[b * N + 2 * k] + I * C_t[b * N + 2 * k + 1];
                    const double complex hn =
                        Abar * (hk[0] + I * hk[1]) + (1.0 - lm) * dl * Abar * up + lm * dl * ut;
                    hk[0] = creal(hn);
                    hk[1] = cimag(hn);
                    acc += creal(conj(ck) * hn);
                }
            } else {
                for (int64_t n = 0; n < N; ++n) {
                    double *hn = &h[(b * D + d) * N + n];
                    const double Abar = exp(dl * A[d * N + n]);
                    *hn = Abar * *hn + (1.0 - lm) * dl * Abar * (B_prev[b * N + n] * xp) +
                          lm * dl * (B_t[b * N + n] * xv);
                    acc += C_t[b * N + n] * *hn;
                }
            }
            y_t[b * D + d] = acc;
        }
    }
    return 0;
}

/*
 * MIMO prefill (scan_chain_mimo, or its complex form when cplx is set): x, y [batch][L][D][R],
 * delta [batch][L][D], B, C [batch][L][N][R], R >= 1.
 */
int oracle_prefill_mimo_f64(const double *x, const double *delta, const double *A, const double *B, const double *C,
                            const double *h0, double *y, double *h_final, int64_t batch, int64_t L, int64_t D,
                            int64_t N, int64_t R, int cplx, int nthreads)
{
    if (R < 1 || (cplx && N % 2 != 0))
        return -1;
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x; j.delta = delta; j.A = A; j.B = B; j.C = C; j.h0 = h0;
    j.y = y; j.h_final = h_final;
    j.batch = batch; j.L = L; j.D = D; j.N = N; j.R = R; j.cplx = cplx;
    return run_scan(j, nthreads);
}

/* One MIMO decode step: h [batch][D][N] in place; x_t, y_t [batch][D][R]; B_t, C_t [batch][N][R]. */
int oracle_step_mimo_f64(double *h, const double *x_t, const double *delta_t, const double *A, const double *B_t,
                         const double *C_t, double *y_t, int64_t batch, int64_t D, int64_t N, int64_t R, int cplx)
{
    /* one token of the prefill is exactly one step: run the chain over L = 1 from h */
    if (R < 1 || (cplx && N % 2 != 0))
        return -1;
    double *hout = (double *)malloc((size_t)(batch * D * N) * sizeof(double));
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x_t; j.delta = delta_t; j.A = A; j.B = B_t; j.C = C_t; j.h0 = h;
    j.y = y_t; j.h_final = hout;
    j.batch = batch; j.L = 1; j.D = D; j.N = N; j.R = R; j.cplx = cplx;
    const int rc = run_scan(j, 1);
    memcpy(h, hout, (size_t)(batch * D * N) * sizeof(double));
    free(hout);
    return rc;
}

/*
 * MIMO prefill with the exponential-trapezoidal rule (scan_chain_mimo with j->trap, or its
 * complex form): lam [batch][L][D]; x_prev [batch][D][R] and B_prev [batch][N][R], both NULL
 * when there is no previous token.
 */
int oracle_prefill_mimo_trapezoid_f64(const double *x, const double *delta, const double *lam, const double *A,
                                      const double *B, const double *C, const double *h0, const double *x_prev,
                                      const double *B_prev, double *y, double *h_final, int64_t batch, int64_t L,
                                      int64_t D, int64_t N, int64_t R, int cplx, int nthreads)
{
    if (R < 1 || (cplx && N % 2 != 0) || ((x_prev == NULL) != (B_prev == NULL)))
        return -1;
    scan_job j;
    memset(&j, 0, sizeof j);
    j.x = x; j.delta = delta; j.A = A; j.B = B; j.C = C; j.h0 = h0;
    j.y = y; j.h_final = h_final;
    j.batch = batch; j.L = L; j.D = D; j.N = N; j.R = R; j.cplx = cplx;
    j.trap = 1; j.lam = lam; j.x_prev = x_prev; j.B_prev = B_prev;
    return run_scan(j, nthreads);
}
