/*
 * ssd_oracle.c -- plain, slow, obviously correct CPU oracle for the complex
 * SSD scan of the Mamba-3-Lite pages.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file. It exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can check and time the GPU path against the
 * plain definition. It shares no code, header or table with the GPU path.
 *
 * What it computes (all arithmetic in double / double complex):
 *
 *   discretisation   -- "Extending" guide, Path A Step 1 (the _discretise
 *                       call) and index.html lab 03 "NAIVE" line:
 *                         Abar_t = exp(softplus(dt_t) * A_h)
 *   recurrence       -- "Extending" guide, Path A Step 1 code block
 *                       (ssd_naive_complex) and index.html lab 03:
 *                         s_t = Abar_t * s_{t-1} + B_t (outer) x_t
 *                         y_t = sum_n C_t[n] * s_t[n, :]
 *                       state s is (N, D) per (batch, head), zero at start;
 *                       no conjugation anywhere (plain products in the code).
 *   per-chunk log-decay -- "Extending" guide, Path B Step 2 and index.html
 *                       lab 03 "CHUNK" line: the inclusive running sum of
 *                       softplus(dt)*A inside each chunk (A_cs).
 *
 * The y output is the full complex y_t; the chunkwise function of the pages
 * returns its real part ("Extending", Path A Step 3), which callers take.
 * final_state is s after the last token t = T-1 (zero-initialised unless an
 * initial state is supplied).
 *
 * softplus is the mathematical log(1 + e^x), evaluated without overflow as
 * max(x, 0) + log1p(exp(-|x|)).
 *
 * Layouts: dense row-major, complex values interleaved (re, im).
 *   x  (B, T, H, D)    Bt, Ct (B, T, H, N)    dt (B, T, H)    A (H)
 *   y  (B, T, H, D)    state  (B, H, N, D)
 *
 * Gradients (oracle_scan_backward) -- reverse-mode differentiation of the same
 * recurrence, for the backward that the "Extending" guide (Path B Step 3, the
 * autograd Function) asks of every scan: true upstream gradients for y and
 * final_state, a gradient for every differentiated input. For a real loss l
 * and a complex input z the gradient is dl/dRe(z) + i dl/dIm(z) (the value
 * torch's autograd stores for complex tensors). The forward states are kept
 * for every step and the adjoint state is walked back from the last token:
 *   lam  <- lam + conj(C_t) (outer) gy_t          (adjoint of s_t)
 *   gC_t = sum_d conj(s_t) gy_t,  gB_t = lam conj(x_t),  gx_t = conj(B_t)^T lam
 *   ga_t = conj(Abar_t) * sum conj(s_{t-1}) lam    (a_t = softplus(dt_t) A)
 *   gdt_t = Re(conj(A) ga_t) * sigmoid(dt_t),  gA += softplus(dt_t) ga_t
 *   lam  <- conj(Abar_t) lam
 * and the gradient of the initial state is the final lam.
 *
 * Parallelism: the (batch, head) sequences are independent; an OpenMP loop
 * runs them side by side. Within a sequence the loop is the plain recurrence.
 */
#include <complex.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Working precision of the recurrence: double for every parity use. A float
 * build (-DORACLE_REAL=float, the pages' complex64) exists only to time the
 * plain recurrence as the CPU baseline; nothing compares against it. */
#ifndef ORACLE_REAL
#define ORACLE_REAL double
#endif
typedef ORACLE_REAL complex cplx;

static double softplus(double v)
{
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

static cplx load_c(const float *p, int64_t i)
{
    return (double)p[2 * i] + I * (double)p[2 * i + 1];
}

static void store_c(double *p, int64_t i, cplx v)
{
    p[2 * i] = creal(v);
    p[2 * i + 1] = cimag(v);
}

int oracle_version(void) { return 3; }

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Abar (B,T,H) and, when chunk > 0, the per-chunk inclusive cumulative
 * log-decay Lambda (B,H,nc,chunk). Positions of the last chunk that lie past
 * T hold the running sum of the last real token (a padded token adds zero). */
int oracle_discretise(const float *dt, const float *A, int64_t Bsz, int64_t T, int64_t H,
                      int64_t chunk, double *A_bar, double *Lambda)
{
    if (!dt || !A || Bsz <= 0 || T <= 0 || H <= 0 || chunk < 0)
        return -1;
    int64_t nc = chunk > 0 ? (T + chunk - 1) / chunk : 0;
    for (int64_t b = 0; b < Bsz; ++b)
        for (int64_t h = 0; h < H; ++h) {
            cplx Ah = load_c(A, h);
            cplx run = 0.0;
            for (int64_t t = 0; t < (chunk > 0 ? nc * chunk : T); ++t) {
                cplx a = 0.0;
                if (t < T)
                    a = softplus((double)dt[(b * T + t) * H + h]) * Ah;
                if (A_bar && t < T)
                    store_c(A_bar, (b * T + t) * H + h, cexp(a));
                if (chunk > 0) {
                    if (t % chunk == 0)
                        run = 0.0;
                    run += a;
                    if (Lambda)
                        store_c(Lambda, ((b * H + h) * nc + t / chunk) * chunk + t % chunk, run);
                }
            }
        }
    return 0;
}

/* The naive O(T) recurrence. y is complex (B,T,H,D); final_state (B,H,N,D).
 * init_state may be NULL (zero state). nthreads <= 0 uses the OpenMP default. */
int oracle_scan(const float *x, const float *A, const float *Bt, const float *Ct, const float *dt,
                int64_t Bsz, int64_t T, int64_t H, int64_t N, int64_t D,
                const double *init_state, double *y, double *final_state, int nthreads)
{
    if (!x || !A || !Bt || !Ct || !dt || Bsz <= 0 || T < 0 || H <= 0 || N <= 0 || D <= 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t nseq = Bsz * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nseq; ++q) {
        int64_t b = q / H, h = q % H;
        cplx *s = malloc(sizeof(cplx) * (size_t)(N * D));
        if (!s) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int64_t i = 0; i < N * D; ++i) {
            int64_t off = (b * H + h) * N * D + i;
            s[i] = init_state ? init_state[2 * off] + I * init_state[2 * off + 1] : 0.0;
        }
        cplx Ah = load_c(A, h);
        for (int64_t t = 0; t < T; ++t) {
            int64_t row = (b * T + t) * H + h;
            cplx Abar = cexp(softplus((double)dt[row]) * Ah);
            /* s = Abar * s + B_t (outer) x_t */
            for (int64_t n = 0; n < N; ++n) {
                cplx bn = load_c(Bt, row * N + n);
                for (int64_t d = 0; d < D; ++d)
                    s[n * D + d] = Abar * s[n * D + d] + bn * load_c(x, row * D + d);
            }
            /* y_t = sum_n C_t[n] * s[n, :] */
            if (y)
                for (int64_t d = 0; d < D; ++d) {
                    cplx acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += load_c(Ct, row * N + n) * s[n * D + d];
                    store_c(y, row * D + d, acc);
                }
        }
        if (final_state)
            for (int64_t i = 0; i < N * D; ++i)
                store_c(final_state, (b * H + h) * N * D + i, s[i]);
        free(s);
    }
    return failed ? -2 : 0;
}

/* Gradients of l = sum_t gy_t . Re(y_t) + sum Re(conj(g_final) * final_state)
 * with respect to x, A, Bt, Ct, dt and the initial state.
 *   grad_y (B,T,H,D) real; grad_final (B,H,N,D) complex or NULL (zero).
 *   gx (B,T,H,D), gB and gC (B,T,H,N), g_init (B,H,N,D) complex; gdt (B,T,H);
 *   gA (H) complex, summed over batch rows in a fixed order.
 * init_state may be NULL (zero); g_init may be NULL. Returns 0, -1 on bad
 * arguments, -2 when memory runs out. */
int oracle_scan_backward(const float *x, const float *A, const float *Bt, const float *Ct,
                         const float *dt, int64_t Bsz, int64_t T, int64_t H, int64_t N, int64_t D,
                         const double *init_state, const float *grad_y, const float *grad_final,
                         double *gx, double *gA, double *gB, double *gC, double *gdt,
                         double *g_init, int nthreads)
{
    if (!x || !A || !Bt || !Ct || !dt || !grad_y || !gx || !gA || !gB || !gC || !gdt ||
        Bsz <= 0 || T < 0 || H <= 0 || N <= 0 || D <= 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t nseq = Bsz * H;
    int64_t ND = N * D;
    cplx *gA_seq = malloc(sizeof(cplx) * (size_t)nseq);
    if (!gA_seq)
        return -2;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nseq; ++q) {
        int64_t b = q / H, h = q % H;
        /* states[t + 1] = s_t, states[0] = the initial state */
        cplx *states = malloc(sizeof(cplx) * (size_t)((T + 1) * ND));
        cplx *lam = malloc(sizeof(cplx) * (size_t)ND);
        if (!states || !lam) {
            free(states);
            free(lam);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int64_t i = 0; i < ND; ++i) {
            int64_t off = (b * H + h) * ND + i;
            states[i] = init_state ? init_state[2 * off] + I * init_state[2 * off + 1] : 0.0;
        }
        cplx Ah = load_c(A, h);
        for (int64_t t = 0; t < T; ++t) {
            int64_t row = (b * T + t) * H + h;
            cplx Abar = cexp(softplus((double)dt[row]) * Ah);
            const cplx *prev = states + t * ND;
            cplx *cur = states + (t + 1) * ND;
            for (int64_t n = 0; n < N; ++n) {
                cplx bn = load_c(Bt, row * N + n);
                for (int64_t d = 0; d < D; ++d)
                    cur[n * D + d] = Abar * prev[n * D + d] + bn * load_c(x, row * D + d);
            }
        }
        for (int64_t i = 0; i < ND; ++i) {
            int64_t off = (b * H + h) * ND + i;
            lam[i] = grad_final ? (double)grad_final[2 * off] + I * (double)grad_final[2 * off + 1]
                                : 0.0;
        }
        cplx gA_acc = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            int64_t row = (b * T + t) * H + h;
            double sp = softplus((double)dt[row]);
            cplx Abar = cexp(sp * Ah);
            const cplx *s_t = states + (t + 1) * ND;
            const cplx *s_prev = states + t * ND;
            /* y_t = Re(sum_n C_t[n] s_t[n, :]) feeds lam with conj(C_t) gy_t */
            for (int64_t n = 0; n < N; ++n) {
                cplx cn = conj(load_c(Ct, row * N + n));
                for (int64_t d = 0; d < D; ++d)
                    lam[n * D + d] += cn * (double)grad_y[row * D + d];
            }
            for (int64_t n = 0; n < N; ++n) {
                cplx acc_c = 0.0, acc_b = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    acc_c += conj(s_t[n * D + d]) * (double)grad_y[row * D + d];
                    acc_b += lam[n * D + d] * conj(load_c(x, row * D + d));
                }
                store_c(gC, row * N + n, acc_c);
                store_c(gB, row * N + n, acc_b);
            }
            for (int64_t d = 0; d < D; ++d) {
                cplx acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += conj(load_c(Bt, row * N + n)) * lam[n * D + d];
                store_c(gx, row * D + d, acc);
            }
            cplx g_abar = 0.0;
            for (int64_t i = 0; i < ND; ++i)
                g_abar += conj(s_prev[i]) * lam[i];
            cplx ga = conj(Abar) * g_abar;
            gdt[row] = creal(conj(Ah) * ga) * sigmoid((double)dt[row]);
            gA_acc += sp * ga;
            for (int64_t i = 0; i < ND; ++i)
                lam[i] = conj(Abar) * lam[i];
        }
        gA_seq[q] = gA_acc;
        if (g_init)
            for (int64_t i = 0; i < ND; ++i)
                store_c(g_init, (b * H + h) * ND + i, lam[i]);
        free(states);
        free(lam);
    }
    for (int64_t h = 0; h < H; ++h) {
        cplx acc = 0.0;
        for (int64_t b = 0; b < Bsz; ++b)
            acc += gA_seq[b * H + h];
        store_c(gA, h, acc);
    }
    free(gA_seq);
    return failed ? -2 : 0;
}

/* MIMO head mixer after the scan -- index.html lab 02 "MIMO MIXER" (a fully
 * connected mixer across the 16 SSM heads, 1024 -> 1024 as 16 heads of 64
 * channels, identity (eye_) at initialisation, 240 off-diagonal head-to-head
 * links), the AGENTS page "Knows cold" item 2, the in_proj -> scan -> MIMO ->
 * out_proj order of the "Extending" guide (Path A), and the model's parameter
 * count in the "Extending" guide's documentation rule (433,662,400, which
 * holds only with a dense 1024 x 1024 matrix in each of the 28 layers).
 * A token's H heads of D channels are flattened head-major, k = h * D + d,
 * and mapped by one dense real F x F matrix (F = H * D), without bias:
 *     z[m, o] = sum_k W[o, k] y[m, k]
 * y, z (M, F) with M = batch * T tokens; W (F, F) row-major (row o holds the
 * weights of output o, as a linear layer stores them). Each block
 * W[i*D:(i+1)*D, j*D:(j+1)*D] is the link from head j to head i. */
int oracle_head_mix(const float *y, const float *W, int64_t M, int64_t H, int64_t D, double *z)
{
    if (!y || !W || !z || M < 0 || H <= 0 || D <= 0)
        return -1;
    const int64_t F = H * D;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t o = 0; o < F; ++o) {
            double acc = 0.0;
            for (int64_t k = 0; k < F; ++k)
                acc += (double)W[o * F + k] * (double)y[m * F + k];
            z[m * F + o] = acc;
        }
    return 0;
}

/* Gradients of l = sum gz * z for the mixer above, by the chain rule on its
 * definition:
 *     gy[m, :] = sum_o gz[m, o] W[o, :]        (gy = W^T gz per token)
 *     gW       = sum_m gz[m, :] (outer) y[m, :]
 * Each sum runs over its index in increasing order; the loops are arranged so
 * that the rows of W and y are read in storage order. Either output may be
 * NULL. */
int oracle_head_mix_backward(const float *y, const float *W, const float *gz, int64_t M,
                             int64_t H, int64_t D, double *gy, double *gW)
{
    if (!y || !W || !gz || M < 0 || H <= 0 || D <= 0)
        return -1;
    const int64_t F = H * D;
    if (gy) {
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            double *row = gy + m * F;
            for (int64_t k = 0; k < F; ++k)
                row[k] = 0.0;
            for (int64_t o = 0; o < F; ++o) {
                const double g = (double)gz[m * F + o];
                for (int64_t k = 0; k < F; ++k)
                    row[k] += g * (double)W[o * F + k];
            }
        }
    }
    if (gW) {
        /* every thread owns whole rows o of gW and adds the outer products
         * token by token */
#pragma omp parallel for schedule(static)
        for (int64_t o = 0; o < F; ++o)
            for (int64_t k = 0; k < F; ++k)
                gW[o * F + k] = 0.0;
#pragma omp parallel
        {
#ifdef _OPENMP
            const int64_t nth = omp_get_num_threads(), me = omp_get_thread_num();
#else
            const int64_t nth = 1, me = 0;
#endif
            const int64_t o0 = F * me / nth, o1 = F * (me + 1) / nth;
            for (int64_t m = 0; m < M; ++m)
                for (int64_t o = o0; o < o1; ++o) {
                    const double g = (double)gz[m * F + o];
                    double *row = gW + o * F;
                    for (int64_t k = 0; k < F; ++k)
                        row[k] += g * (double)y[m * F + k];
                }
        }
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
