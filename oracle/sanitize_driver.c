/*
 * Host driver for the sanitizer check of the oracle (test infrastructure,
 * like the oracle itself).  Built with -fsanitize=address,undefined together
 * with mdn_oracle.c by tests/test_oracle_sanitized.py and run as a process
 * of its own: it calls every exported function of the oracle on small and
 * degenerate shapes (no tokens, one token, ragged column blocks, absent
 * optional arrays, chunk lengths that do and do not divide T) and on the
 * argument errors, so that any out-of-bounds access, leak or undefined
 * operation in them stops the process.  Prints "ok" on success.
 */
#include <stdio.h>
#include <stdlib.h>

int mdn_oracle_recurrence(const double* q, const double* k, const double* v,
                          const double* alpha, const double* beta, const double* mu,
                          const double* eta, const double* S0, const double* M0, double* O,
                          double* ST, double* MT, int B, int T, int H, int Dk, int Dv,
                          int col_block, int nthreads);
int mdn_oracle_recurrence_vt(const double* q, const double* k, const double* v,
                             const double* alpha, const double* beta, const double* mu,
                             const double* eta, const double* S0, const double* M0, double* O,
                             double* ST, double* MT, double* VT, int B, int T, int H, int Dk,
                             int Dv, int col_block, int nthreads);
int mdn_oracle_recurrence_backward(const double* q, const double* k, const double* v,
                                   const double* alpha, const double* beta, const double* mu,
                                   const double* eta, const double* S0, const double* M0,
                                   const double* dO, const double* dST, const double* dMT,
                                   double* dq, double* dk, double* dv, double* dalpha,
                                   double* dbeta, double* dmu, double* deta, double* dS0,
                                   double* dM0, int B, int T, int H, int Dk, int Dv,
                                   int col_block, int nthreads);
int mdn_oracle_chunk_bruteforce(const double* q, const double* k, const double* v,
                                const double* alpha, const double* beta, const double* mu,
                                const double* eta, const double* S0, const double* M0,
                                double* O, double* ST, double* MT, int B, int T, int H, int Dk,
                                int Dv, int C, int gamma_form, int flags);
int mdn_oracle_chunk_gamma(const double* alpha, const double* beta, const double* mu, int n,
                           int form, double* G);
int mdn_oracle_max_threads(void);

static unsigned long long rng_state = 0x9e3779b97f4a7c15ull;

/* uniform in [lo, hi) from a 64-bit linear congruential generator */
static double uni(double lo, double hi)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (double)(rng_state >> 11) / 9007199254740992.0;
}

/* a buffer of n doubles (at least one, so that an empty shape still has a
 * valid pointer) filled from [lo, hi) */
static double* buf(size_t n, double lo, double hi)
{
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    for (size_t i = 0; i < (n ? n : 1); ++i) p[i] = uni(lo, hi);
    return p;
}

static int fail(const char* what, int rc)
{
    fprintf(stderr, "%s returned %d\n", what, rc);
    return 1;
}

int main(void)
{
    static const int shapes[][5] = {{1, 0, 1, 4, 4}, {1, 1, 1, 3, 5}, {2, 7, 3, 4, 6},
                                    {1, 9, 2, 5, 3}, {2, 16, 1, 8, 8}};
    static const int col_blocks[] = {0, 1, 2, 5, 64};
    int bad = 0;
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int B = shapes[s][0], T = shapes[s][1], H = shapes[s][2], Dk = shapes[s][3],
                  Dv = shapes[s][4];
        const size_t nk = (size_t)B * T * H * Dk, nv = (size_t)B * T * H * Dv,
                     ng = (size_t)B * T * H, ns = (size_t)B * H * Dk * Dv;
        double *q = buf(nk, -1, 1), *k = buf(nk, -1, 1), *v = buf(nv, -1, 1);
        double *al = buf(ng, 0.5, 1), *be = buf(ng, 0.2, 1), *mu = buf(ng, 0, 0.9),
               *et = buf(ng, 0.05, 0.5);
        double *S0 = buf(ns, -0.3, 0.3), *M0 = buf(ns, -0.3, 0.3);
        double *O = buf(nv, 0, 0), *ST = buf(ns, 0, 0), *MT = buf(ns, 0, 0), *VT = buf(nv, 0, 0);
        double *dO = buf(nv, -1, 1), *dST = buf(ns, -1, 1), *dMT = buf(ns, -1, 1);
        double *dq = buf(nk, 0, 0), *dk = buf(nk, 0, 0), *dv = buf(nv, 0, 0), *da = buf(ng, 0, 0),
               *db = buf(ng, 0, 0), *dm = buf(ng, 0, 0), *de = buf(ng, 0, 0), *dS = buf(ns, 0, 0),
               *dM = buf(ns, 0, 0);
        for (size_t c = 0; c < sizeof(col_blocks) / sizeof(col_blocks[0]); ++c) {
            const int cb = col_blocks[c];
            for (int opt = 0; opt < 4; ++opt) {
                const double* beta = opt & 1 ? be : NULL;
                const double* s0 = opt & 2 ? S0 : NULL;
                const double* m0 = opt & 2 ? M0 : NULL;
                int rc = mdn_oracle_recurrence(q, k, v, al, beta, mu, et, s0, m0, O, ST, MT, B, T,
                                               H, Dk, Dv, cb, 2);
                if (rc) bad |= fail("recurrence", rc);
                rc = mdn_oracle_recurrence_vt(q, k, v, al, beta, mu, et, s0, m0, O, ST, MT, VT, B,
                                              T, H, Dk, Dv, cb, 2);
                if (rc) bad |= fail("recurrence_vt", rc);
                rc = mdn_oracle_recurrence_backward(q, k, v, al, beta, mu, et, s0, m0, dO,
                                                    opt & 2 ? dST : NULL, opt & 2 ? dMT : NULL,
                                                    dq, dk, dv, da, beta ? db : NULL, dm, de,
                                                    opt & 1 ? dS : NULL, opt & 1 ? dM : NULL, B,
                                                    T, H, Dk, Dv, cb, 2);
                if (rc) bad |= fail("recurrence_backward", rc);
            }
        }
        for (int C = 1; C <= 8; ++C)
            for (int form = 0; form < 3; ++form)
                for (int flags = 0; flags < 8; ++flags) {
                    const int rc = mdn_oracle_chunk_bruteforce(q, k, v, al, flags & 1 ? be : NULL,
                                                               mu, et, S0, M0, O, ST, MT, B, T, H,
                                                               Dk, Dv, C, form, flags);
                    if (rc) bad |= fail("chunk_bruteforce", rc);
                }
        /* argument errors return codes and touch nothing */
        if (mdn_oracle_recurrence(NULL, k, v, al, NULL, mu, et, NULL, NULL, O, ST, MT, B, T, H, Dk,
                                  Dv, 0, 1) == 0)
            bad |= fail("recurrence without q", 0);
        if (mdn_oracle_recurrence_vt(q, k, v, al, NULL, mu, et, NULL, NULL, O, ST, MT, NULL, B, T,
                                     H, Dk, Dv, 0, 1) == 0)
            bad |= fail("recurrence_vt without VT", 0);
        if (mdn_oracle_recurrence_backward(q, k, v, al, NULL, mu, et, NULL, NULL, NULL, NULL, NULL,
                                           dq, dk, dv, da, NULL, dm, de, NULL, NULL, B, T, H, Dk,
                                           Dv, 0, 1) == 0)
            bad |= fail("backward without dO", 0);
        if (mdn_oracle_chunk_bruteforce(q, k, v, al, NULL, mu, et, NULL, NULL, O, ST, MT, B, T, H,
                                        Dk, Dv, 0, 0, 0) == 0)
            bad |= fail("bruteforce with C = 0", 0);
        double* ptrs[] = {q, k, v, al, be, mu, et, S0, M0, O, ST, MT, VT, dO, dST, dMT,
                          dq, dk, dv, da, db, dm, de, dS, dM};
        for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) free(ptrs[i]);
    }
    for (int n = 1; n <= 9; n += 4)
        for (int form = 0; form < 3; ++form) {
            double *al = buf(n, 0.5, 1), *be = buf(n, 0.2, 1), *mu = buf(n, 0, 0.9);
            double* G = buf((size_t)n * n, 0, 0);
            int rc = mdn_oracle_chunk_gamma(al, be, mu, n, form, G);
            if (rc) bad |= fail("chunk_gamma", rc);
            rc = mdn_oracle_chunk_gamma(al, NULL, mu, n, form, G);
            if (rc) bad |= fail("chunk_gamma without beta", rc);
            free(al);
            free(be);
            free(mu);
            free(G);
        }
    if (mdn_oracle_max_threads() < 1) bad |= fail("max_threads", 0);
    if (bad) return 1;
    printf("ok\n");
    return 0;
}
