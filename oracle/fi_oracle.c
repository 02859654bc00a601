/*
 * fi_oracle.c -- CPU oracle for the exact online causal long convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the GPU path.
 *
 * Source: the page "Flash Inference: Inferenza in Tempo Quasi-Lineare per
 * Modelli di Sequenza a Convoluzione Lunga e Oltre" (lowest.today summary of
 * arXiv 2410.12982), written [FI] below.
 *
 * What it computes is the plain definition, not the method: the method (the
 * relaxed tiling of [FI] "Strategia di Tiling (Algoritmo 1)") reaches the same
 * sums exactly up to rounding order, so the oracle is the definition written
 * out, in fp64, with every sum taken in ascending input position.
 *
 * Conventions (0-indexed restatement of [FI] "Definizione del Compito" and
 * "Definizione Specifica di LCSM"): channels are (b, c) with b in [0,B),
 * c in [0,D); the filter h[j][c] (j in [0,L)) is shared across b; layouts are
 * row-major with channels innermost: h[L][D], x[B][L][D], y[B][L][D].
 *
 *   y[b][t][c] = sum_{s=0}^{t} h[t-s][c] * x[b][s][c]        (lag 0 included)
 *
 * Closed loop: x[b][0][c] is given and, after y[b][t][c] is known,
 * x[b][t+1][c] = tanh(y[b][t][c]) (the per-channel feedback that stands in for
 * the model's block and sampler of [FI] "Algoritmo di Inferenza LCSM
 * (Algoritmo 2)"); with bf16 storage the fed-back value is rounded to bf16,
 * nearest-even.
 *
 * Prompted: the generation task of [FI] "Definizione del Compito" starts from
 * a prompt x_1 .. x_p.  Here x[b][s][c] is given for s < p and fed back,
 * x[b][t+1][c] = tanh(y[b][t][c]), from position p on.  p = 1 is the closed
 * loop and p = L the open loop.
 *
 * Mutation hooks: building with -DFIO_MUTANT=k plants one deliberate mistake
 * (k = 1..12, listed at each hook; 8..12 are in the multi-layer stack).  The test suite builds every mutant on the
 * CPU and checks that each one fails at least one pin; the normal build never
 * defines FIO_MUTANT.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef FIO_MUTANT
#define FIO_MUTANT 0
#endif

/* Channels processed together by one thread: the innermost loop runs over
 * them so it vectorises without reassociating any single channel's sum. */
#define FIO_CBLK 16

/* Round a double to the nearest bf16 value (8 significant bits), ties to
 * even.  Exact: scaling by a power of two and rint() (round-half-even under
 * the default rounding mode) introduce no other rounding. */
double fio_round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e2;
    frexp(v, &e2);                 /* |v| in [2^(e2-1), 2^e2) */
    int e = e2 - 1;
    if (e < -126) e = -126;        /* bf16 subnormal range: fixed quantum */
    double q = ldexp(1.0, e - 7);  /* weight of the last kept bit */
#if FIO_MUTANT == 6
    return floor(v / q) * q;       /* mutant 6: truncation instead of nearest-even */
#else
    return rint(v / q) * q;
#endif
}

/* One batch element, channels [c0, c0+cn), all positions.  x[s][.] is read
 * for s < p; for t + 1 >= p, x[t+1][.] is written from tanh(y[t][.]) (p = L:
 * open loop, p = 1: closed loop). */
static void conv_block(int64_t D, int64_t L, int64_t c0, int64_t cn,
                       const double *h, double *x, double *y,
                       int64_t p, int round_bf16)
{
    double acc[FIO_CBLK];
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t k = 0; k < cn; ++k) acc[k] = 0.0;
#if FIO_MUTANT == 1
        for (int64_t s = 0; s < t; ++s) {          /* mutant 1: lag-0 term dropped */
#else
        for (int64_t s = 0; s <= t; ++s) {
#endif
#if FIO_MUTANT == 2
            const double *hr = h + (t - s + (t > s ? 1 : 0)) % L * D + c0;  /* mutant 2: lag off by one */
#elif FIO_MUTANT == 3
            const double *hr = h + s * D + c0;    /* mutant 3: filter index s instead of t-s */
#else
            const double *hr = h + (t - s) * D + c0;
#endif
            const double *xr = x + s * D + c0;
            for (int64_t k = 0; k < cn; ++k) {
#if FIO_MUTANT == 4
                acc[k] += hr[(k + 1) % cn] * xr[k];  /* mutant 4: neighbouring channel's filter */
#else
                acc[k] += hr[k] * xr[k];
#endif
            }
        }
        double *yr = y + t * D + c0;
        for (int64_t k = 0; k < cn; ++k) yr[k] = acc[k];
#if FIO_MUTANT == 7
        if (t + 2 >= p && t + 1 < L) {  /* mutant 7: feedback starts one position early */
#else
        if (t + 1 >= p && t + 1 < L) {
#endif
            double *xn = x + (t + 1) * D + c0;
            for (int64_t k = 0; k < cn; ++k) {
#if FIO_MUTANT == 5
                double f = tanh(acc[k]) * 0.5;     /* mutant 5: wrong feedback */
#else
                double f = tanh(acc[k]);
#endif
                xn[k] = round_bf16 ? fio_round_bf16(f) : f;
            }
        }
    }
}

static void run(int64_t B, int64_t D, int64_t L, const double *h, double *x,
                double *y, int64_t p, int round_bf16, int nthreads)
{
    int64_t nblk = (D + FIO_CBLK - 1) / FIO_CBLK;
    int64_t jobs = B * nblk;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t j = 0; j < jobs; ++j) {
        int64_t b = j / nblk, c0 = (j % nblk) * FIO_CBLK;
        int64_t cn = D - c0 < FIO_CBLK ? D - c0 : FIO_CBLK;
        conv_block(D, L, c0, cn, h, x + b * L * D, y + b * L * D,
                   p, round_bf16);
    }
    (void)nthreads;
}

/* Open loop: y = causal convolution of x with h, every channel, every position. */
void fio_open(int64_t B, int64_t D, int64_t L, const double *h,
              const double *x, double *y, int nthreads)
{
    run(B, D, L, h, (double *)x, y, L, 0, nthreads);
}

/* Closed loop, free-running.  x_io[B][L][D]: on entry x_io[b][0][c] holds x0;
 * on return every x_io[b][t][c] holds the input that produced y[b][t][c]. */
void fio_closed(int64_t B, int64_t D, int64_t L, const double *h, double *x_io,
                double *y, int round_bf16, int nthreads)
{
    run(B, D, L, h, x_io, y, 1, round_bf16, nthreads);
}

/* Prompted, free-running after the prompt.  x_io[B][L][D]: on entry
 * x_io[b][s][c] holds the prompt for s < p (1 <= p <= L); on return every
 * x_io[b][t][c] holds the input that produced y[b][t][c]. */
void fio_prompted(int64_t B, int64_t D, int64_t L, int64_t p, const double *h,
                  double *x_io, double *y, int round_bf16, int nthreads)
{
    run(B, D, L, h, x_io, y, p, round_bf16, nthreads);
}

/* One channel, selected positions: y_k = sum_{s=0}^{t_k} h[t_k - s] x[s],
 * with h and x given as that channel's series of length L. */
void fio_points(int64_t L, const double *h, const double *x, int64_t n,
                const int64_t *t, double *y)
{
    for (int64_t k = 0; k < n; ++k) {
        int64_t tk = t[k];
        double acc = 0.0;
        if (tk >= 0 && tk < L)
            for (int64_t s = 0; s <= tk; ++s) acc += h[tk - s] * x[s];
        y[k] = acc;
    }
}

/* ------------------------------------------------------------------ stack
 * The multi-layer LCSM of [FI] "Algoritmo di Inferenza LCSM (Algoritmo 2)"
 * and "Architettura del Modello" (a_i of layer l = block_l(mixer_l(a of layer
 * l-1)_i)), with the synthetic blocks of [FI] "Configurazione Sperimentale"
 * (MLP + GELU) and a sampler that adds given noise, 0-indexed: layers
 * l = 0..M-1, a^0 = x (the stack's input sequence), and for every position t
 *
 *   z^l_t[c]   = sum_{s=0}^{t} rho^l[t-s][c] * a^l_s[c]         (the mixer)
 *   a^{l+1}_t  = W2^l act(W1^l z^l_t)                           (the block)
 *   x_{t+1}    = a^M_t + sigma * noise[t]                       (the sampler)
 *
 * act(v) = GELU(v) = v (1 + erf(v / sqrt 2)) / 2 (act_kind 0), tanh (1) or
 * the identity (2); W1^l, W2^l are D x D, row j holding the weights of
 * output j.  teacher_forced != 0: x is given at every position and only y is
 * computed; otherwise x[0] is given and the rest is fed back.  Layouts:
 * rho[M][L][D], w1 and w2 [M][D][D], x, noise (or NULL), y [B][L][D]; y
 * receives a^M.  Plain fp64, every sum in ascending index. */
static double act_fn(double v, int kind)
{
#if FIO_MUTANT == 11
    if (kind == 0)   /* mutant 11: the tanh approximation of GELU */
        return 0.5 * v * (1.0 + tanh(0.7978845608028654 * (v + 0.044715 * v * v * v)));
#endif
    if (kind == 0) return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
    if (kind == 1) return tanh(v);
    return v;
}

static void stack_row(int64_t D, int64_t L, int64_t M, const double *rho, const double *w1,
                      const double *w2, double *x, const double *noise, double sigma, int act_kind,
                      int teacher_forced, double *y, double *a /* [M+1][L][D] work */,
                      double *z /* [D] */, double *hb /* [D] */)
{
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t c = 0; c < D; ++c) a[t * D + c] = x[t * D + c];   /* a^0_t */
        for (int64_t l = 0; l < M; ++l) {
#if FIO_MUTANT == 9
            const double *r = rho;                         /* mutant 9: layer 0's filter everywhere */
#else
            const double *r = rho + l * L * D;
#endif
            const double *al = a + l * L * D;
            for (int64_t c = 0; c < D; ++c) {
                double acc = 0.0;
                for (int64_t s = 0; s <= t; ++s) acc += r[(t - s) * D + c] * al[s * D + c];
                z[c] = acc;
            }
            const double *W1 = w1 + l * D * D, *W2 = w2 + l * D * D;
            double *an = a + (l + 1) * L * D + t * D;
#if FIO_MUTANT == 8
            /* mutant 8: both products before the activation */
            for (int64_t j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < D; ++k) acc += W1[j * D + k] * z[k];
                hb[j] = acc;
            }
            for (int64_t j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < D; ++k) acc += W2[j * D + k] * hb[k];
                an[j] = act_fn(acc, act_kind);
            }
#else
            for (int64_t j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < D; ++k) acc += W1[j * D + k] * z[k];
                hb[j] = act_fn(acc, act_kind);
            }
            for (int64_t j = 0; j < D; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < D; ++k) acc += W2[j * D + k] * hb[k];
#if FIO_MUTANT == 12
                an[j] = z[j];                              /* mutant 12: the next layer reads the mixer output */
                (void)acc;
#else
                an[j] = acc;
#endif
            }
#endif
        }
        const double *aM = a + M * L * D + t * D;
        for (int64_t c = 0; c < D; ++c) y[t * D + c] = aM[c];
        if (!teacher_forced && t + 1 < L) {
            for (int64_t c = 0; c < D; ++c) {
#if FIO_MUTANT == 10
                const double nz = noise && t + 1 < L ? noise[(t + 1) * D + c] : 0.0;  /* mutant 10: noise of t+1 */
#else
                const double nz = noise ? noise[t * D + c] : 0.0;
#endif
                x[(t + 1) * D + c] = aM[c] + sigma * nz;
            }
        }
    }
}

/* The stack over B batch rows (independent; the weights and filters are
 * shared).  work: [B][(M+1) L D + 2 D] doubles supplied by the caller. */
void fio_stack(int64_t B, int64_t D, int64_t L, int64_t M, const double *rho, const double *w1,
               const double *w2, double *x, const double *noise, double sigma, int act_kind,
               int teacher_forced, double *y, double *work, int nthreads)
{
    const int64_t wsz = (M + 1) * L * D + 2 * D;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t b = 0; b < B; ++b) {
        double *wk = work + b * wsz;
        stack_row(D, L, M, rho, w1, w2, x + b * L * D, noise ? noise + b * L * D : NULL, sigma, act_kind,
                  teacher_forced, y + b * L * D, wk, wk + (M + 1) * L * D, wk + (M + 1) * L * D + D);
    }
    (void)nthreads;
}

int fio_mutant(void) { return FIO_MUTANT; }
