/* Test infrastructure: runs every entry point of the oracle (oracle/fi_oracle.c)
 * on small seeded inputs, edge arguments included, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer checks its memory accesses
 * and arithmetic.  It prints a checksum and returns 0; the sanitizers abort
 * on the first finding. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double fio_round_bf16(double v);
void fio_open(int64_t B, int64_t D, int64_t L, const double *h, const double *x, double *y, int nthreads);
void fio_closed(int64_t B, int64_t D, int64_t L, const double *h, double *x_io, double *y, int round_bf16,
                int nthreads);
void fio_prompted(int64_t B, int64_t D, int64_t L, int64_t p, const double *h, double *x_io, double *y,
                  int round_bf16, int nthreads);
void fio_points(int64_t L, const double *h, const double *x, int64_t n, const int64_t *t, double *y);
void fio_stack(int64_t B, int64_t D, int64_t L, int64_t M, const double *rho, const double *w1, const double *w2,
               double *x, const double *noise, double sigma, int act_kind, int teacher_forced, double *y,
               double *work, int nthreads);

static unsigned seed = 12345u;

/* exactly-sized arrays (so an access one past the end is caught) of values in [-1, 1) */
static double *draw(int64_t n) {
    double *p = malloc((size_t)n * sizeof *p);
    for (int64_t i = 0; i < n; ++i) {
        seed = seed * 1103515245u + 12345u;
        p[i] = (double)((seed >> 8) & 0xFFFF) / 32768.0 - 1.0;
    }
    return p;
}

static double *copy(const double *a, int64_t n) {
    double *p = malloc((size_t)n * sizeof *p);
    memcpy(p, a, (size_t)n * sizeof *p);
    return p;
}

static double sum(const double *a, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += a[i];
    return s;
}

int main(void) {
    const int64_t B = 2, D = 3, L = 37, M = 2, N = B * L * D;
    double check = 0.0;
    double *h = draw(L * D), *x = draw(N), *y = malloc((size_t)N * sizeof *y);

    fio_open(B, D, L, h, x, y, 1);
    check += sum(y, N);
    fio_open(1, 1, 1, h, x, y, 1);   /* the smallest problem */
    check += y[0];
    for (int bf = 0; bf < 2; ++bf) {
        double *xio = copy(x, N);
        fio_closed(B, D, L, h, xio, y, bf, 1);
        check += sum(y, N) + sum(xio, N);
        free(xio);
    }
    const int64_t prompts[] = {1, 2, 36, L};
    for (int k = 0; k < 4; ++k) {
        double *xio = copy(x, N);
        fio_prompted(B, D, L, prompts[k], h, xio, y, k & 1, 1);
        check += sum(y, N);
        free(xio);
    }
    /* positions outside [0, L) give 0 */
    const int64_t ts[] = {0, 1, L - 1, -1, L};
    double yp[5];
    double *hc = malloc((size_t)L * sizeof *hc), *xc = malloc((size_t)L * sizeof *xc);
    for (int64_t t = 0; t < L; ++t) {
        hc[t] = h[t * D];
        xc[t] = x[t * D];
    }
    fio_points(L, hc, xc, 5, ts, yp);
    check += sum(yp, 5);

    double *rho = draw(M * L * D), *w1 = draw(M * D * D), *w2 = draw(M * D * D), *nz = draw(N);
    double *work = malloc((size_t)(B * ((M + 1) * L * D + 2 * D)) * sizeof *work);
    for (int act = 0; act < 3; ++act)
        for (int tf = 0; tf < 2; ++tf) {
            double *xs = copy(x, N);
            fio_stack(B, D, L, M, rho, w1, w2, xs, act == 1 ? NULL : nz, 0.25, act, tf, y, work, 1);
            check += sum(y, N) + sum(xs, N);
            free(xs);
        }

    const double vals[] = {0.0, -0.0, 1.0, 1.00390625, 1.0 + 1.0 / 256.0 + 1e-9, 3.0e38, -1.0e-40};
    for (int k = 0; k < 7; ++k) check += fio_round_bf16(vals[k]) * 1e-38;

    printf("checksum %.17g\n", check);
    free(h); free(x); free(y); free(hc); free(xc); free(rho); free(w1); free(w2); free(nz); free(work);
    return 0;
}
