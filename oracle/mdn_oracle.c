/*
 * mdn_oracle.c -- fp64 CPU oracle for Momentum DeltaNet (MDN).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent, slow, obviously
 * correct reference that the GPU library is checked against.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library, and the
 * HIP library never calls it: there is no CPU fallback anywhere.
 *
 * Sources (the pages this follows):
 *   [MDN slides]  "MDN: Parallelizing Stepwise Momentum for Delta Linear
 *                 Attention" (slides, with backup frames on formula errata)
 *   [MDN notes]   reading notes on the same paper (Chinese), Secs. 2.2-2.5
 *
 * Two independent computations live here:
 *
 *   mdn_oracle_recurrence   the token-by-token two-state recurrence,
 *                           [MDN slides] Sec. 3.1 Eqs. (3)-(5) and
 *                           [MDN notes] Sec. 2.2 (boxed update).  This is THE
 *                           oracle: the chunkwise form is an exact algebraic
 *                           rewrite of it ([MDN slides] "Chunk outputs combine
 *                           incoming states and local writes"), so the
 *                           recurrence itself defines the right answer.
 *
 *   mdn_oracle_chunk_bruteforce
 *                           a literal fp64 evaluation of the chunkwise
 *                           equations ([MDN slides] Eqs. (7)-(9), (15)-(18),
 *                           (40)-(42) with the Appendix C/E corrections;
 *                           [MDN notes] Secs. 2.3-2.5), with Gamma from its
 *                           product-sum definition and T from a Gauss-Jordan
 *                           inverse.  Used only on tiny inputs to cross-check
 *                           the recurrence and the chunk algebra.
 *
 * Every floating-point value is double.  beta may be NULL, meaning beta == 1
 * at every token (the library's fixed semantics); the oracle keeps the gate
 * so that the general four-gate form can be checked.
 *
 * Layouts (row-major, C order):
 *   q, k        [B, T, H, Dk]
 *   v, O        [B, T, H, Dv]
 *   gates       [B, T, H]          (alpha, beta, mu, eta)
 *   S0,M0,ST,MT [B, H, Dk, Dv]     (S0/M0 may be NULL: zero initial state;
 *                                   ST/MT may be NULL: not returned)
 */
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_TOK(b, t, h, d, T, H, D) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (D) + (d))
#define IDX_GATE(b, t, h, T, H) (((size_t)(b) * (T) + (t)) * (H) + (h))
#define IDX_STATE(b, h, i, c, H, Dk, Dv) ((((size_t)(b) * (H) + (h)) * (Dk) + (i)) * (Dv) + (c))

/* ------------------------------------------------------------------------ */
/* Token recurrence                                                          */
/* ------------------------------------------------------------------------ */

/* One token's update of a column block of S and M, in place (the step
 * recurrence_unit describes); vt receives the residual. */
static void token_step(const double* kt, const double* vv, double a, double m, double e,
                       double s, double* S, double* M, double* vt, int Dk, int nc)
{
    /* S_{t-1}^T k_t, column by column */
    for (int c = 0; c < nc; ++c) vt[c] = 0.0;
    for (int i = 0; i < Dk; ++i)
        for (int c = 0; c < nc; ++c) vt[c] += S[(size_t)i * nc + c] * kt[i];
    for (int c = 0; c < nc; ++c) vt[c] = vv[c] - a * vt[c];

    /* momentum, then memory (which reads the new momentum) */
    for (int i = 0; i < Dk; ++i) {
        for (int c = 0; c < nc; ++c) {
            const size_t x = (size_t)i * nc + c;
            M[x] = m * M[x] - e * kt[i] * vt[c];
            S[x] = a * S[x] - s * M[x];
        }
    }
}

/*
 * One (b, h, column block) work unit.  Columns of S and M evolve
 * independently given q, k and the gates: every step below acts on each
 * column c separately (the residual, the momentum and memory updates and the
 * read-out are all column-wise), so the d_v axis can be split freely.
 *
 * For t = 1..T, with a = alpha_t, m = mu_t, e = eta_t, s = beta_t:
 *     vt  = v_t - a * S_{t-1}^T k_t          residual against the decayed memory
 *     M_t = m * M_{t-1} - e * k_t vt^T       momentum accumulates the gradient
 *     S_t = a * S_{t-1} - s * M_t            memory moves along the momentum
 *     o_t = S_t^T q_t                        read-out uses the updated memory
 * ([MDN slides] Sec. 3.1 Eqs. (3)-(5); [MDN notes] Sec. 2.2.)
 */
static void recurrence_unit(const double* q, const double* k, const double* v,
                            const double* alpha, const double* beta, const double* mu,
                            const double* eta, const double* S0, const double* M0,
                            double* O, double* ST, double* MT, double* VT, int b, int h, int c0,
                            int nc,
                            int T, int H, int Dk, int Dv, double* S, double* M, double* vt,
                            double* o)
{
    for (int i = 0; i < Dk; ++i) {
        for (int c = 0; c < nc; ++c) {
            S[(size_t)i * nc + c] = S0 ? S0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;
            M[(size_t)i * nc + c] = M0 ? M0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;
        }
    }
    for (int t = 0; t < T; ++t) {
        const size_t g = IDX_GATE(b, t, h, T, H);
        const double a = alpha[g];
        const double m = mu[g];
        const double e = eta[g];
        const double s = beta ? beta[g] : 1.0;
        const double* kt = k + IDX_TOK(b, t, h, 0, T, H, Dk);
        const double* qt = q + IDX_TOK(b, t, h, 0, T, H, Dk);
        const double* vv = v + IDX_TOK(b, t, h, c0, T, H, Dv);

        token_step(kt, vv, a, m, e, s, S, M, vt, Dk, nc);

        /* o_t = S_t^T q_t */
        for (int c = 0; c < nc; ++c) o[c] = 0.0;
        for (int i = 0; i < Dk; ++i)
            for (int c = 0; c < nc; ++c) o[c] += S[(size_t)i * nc + c] * qt[i];
        double* ot = O + IDX_TOK(b, t, h, c0, T, H, Dv);
        for (int c = 0; c < nc; ++c) ot[c] = o[c];
        if (VT) {
            double* vo = VT + IDX_TOK(b, t, h, c0, T, H, Dv);
            for (int c = 0; c < nc; ++c) vo[c] = vt[c];
        }
    }
    for (int i = 0; i < Dk; ++i) {
        for (int c = 0; c < nc; ++c) {
            if (ST) ST[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] = S[(size_t)i * nc + c];
            if (MT) MT[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] = M[(size_t)i * nc + c];
        }
    }
}

/*
 * Full recurrence over [B, T, H].  col_block <= 0 means one block of Dv
 * columns.  nthreads <= 0 leaves OpenMP's default.  Returns 0 on success,
 * nonzero on bad arguments or allocation failure.
 */
static int recurrence_all(const double* q, const double* k, const double* v,
                          const double* alpha, const double* beta, const double* mu,
                          const double* eta, const double* S0, const double* M0, double* O,
                          double* ST, double* MT, double* VT, int B, int T, int H, int Dk,
                          int Dv, int col_block, int nthreads)
{
    if (!q || !k || !v || !alpha || !mu || !eta || !O) return 1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return 2;
    if (col_block <= 0 || col_block > Dv) col_block = Dv;
    const int nblk = (Dv + col_block - 1) / col_block;
    const long units = (long)B * H * nblk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : failed)
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)Dk * col_block);
        double* M = (double*)malloc(sizeof(double) * (size_t)Dk * col_block);
        double* vt = (double*)malloc(sizeof(double) * (size_t)col_block);
        double* o = (double*)malloc(sizeof(double) * (size_t)col_block);
        const int ok = S && M && vt && o;
        if (!ok) failed = 1;
        /* every thread reaches the work-sharing loop, even one whose
         * allocation failed (it then takes no work) */
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!ok) continue;
            const int blk = (int)(u % nblk);
            const int h = (int)((u / nblk) % H);
            const int b = (int)(u / ((long)nblk * H));
            const int c0 = blk * col_block;
            const int nc = (c0 + col_block <= Dv) ? col_block : Dv - c0;
            recurrence_unit(q, k, v, alpha, beta, mu, eta, S0, M0, O, ST, MT, VT, b, h, c0, nc, T,
                            H, Dk, Dv, S, M, vt, o);
        }
        free(S);
        free(M);
        free(vt);
        free(o);
    }
    return failed ? 3 : 0;
}

int mdn_oracle_recurrence(const double* q, const double* k, const double* v,
                          const double* alpha, const double* beta, const double* mu,
                          const double* eta, const double* S0, const double* M0, double* O,
                          double* ST, double* MT, int B, int T, int H, int Dk, int Dv,
                          int col_block, int nthreads)
{
    return recurrence_all(q, k, v, alpha, beta, mu, eta, S0, M0, O, ST, MT, NULL, B, T, H, Dk,
                          Dv, col_block, nthreads);
}

/* The same recurrence, also returning every token's residual vt_t [B,T,H,Dv]
 * (the quantity the chunk form calls Vt). */
int mdn_oracle_recurrence_vt(const double* q, const double* k, const double* v,
                             const double* alpha, const double* beta, const double* mu,
                             const double* eta, const double* S0, const double* M0, double* O,
                             double* ST, double* MT, double* VT, int B, int T, int H, int Dk,
                             int Dv, int col_block, int nthreads)
{
    if (!VT) return 1;
    return recurrence_all(q, k, v, alpha, beta, mu, eta, S0, M0, O, ST, MT, VT, B, T, H, Dk, Dv,
                          col_block, nthreads);
}

/* Number of threads OpenMP would use for a parallel region (for reporting). */
int mdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Reverse-mode derivative of the token recurrence                           */
/* ------------------------------------------------------------------------ */

/*
 * The pages give the backward pass's strategy but no gradient formulas, so
 * this is the plain reverse-mode derivative of the recurrence above (the
 * chain rule applied to each line of the token step, last token first).
 * Given dO = dL/dO, dST = dL/dS_T and dMT = dL/dM_T, and writing Sh and Mh for
 * the running gradients dL/dS_t and dL/dM_t (from the later tokens), token t
 * (a = alpha_t, m = mu_t, e = eta_t, s = beta_t) contributes:
 *     o_t = S_t^T q_t:              Sh += q_t do_t^T;  dq_t = S_t do_t
 *     S_t = a S_{t-1} - s M_t:      dalpha_t += <S_{t-1}, Sh>;  dbeta_t = -<M_t, Sh>
 *                                   P = Mh - s Sh  (the whole dL/dM_t)
 *     M_t = m M_{t-1} - e k_t vt^T: dmu_t = <M_{t-1}, P>;  deta_t = -k_t^T P vt
 *                                   dk_t = -e P vt;  dvt = -e P^T k_t
 *     vt = v_t - a S_{t-1}^T k_t:   dv_t = dvt;  dk_t += -a S_{t-1} dvt
 *                                   dalpha_t += -k_t^T S_{t-1} dvt
 * and hands on Sh <- a Sh - a k_t dvt^T, Mh <- m P.  After token 1,
 * dS0 = Sh and dM0 = Mh.  <X, Y> is the sum of X .* Y over d_k x d_v.
 *
 * A work unit is one (b, h); it runs column blocks one after another, each
 * with its forward states S_t, M_t (t = 0..T) stored, and adds the column
 * sums (dq, dk and the gate gradients) into the unit's own slices.
 */
static void backward_unit(const double* q, const double* k, const double* v,
                          const double* alpha, const double* beta, const double* mu,
                          const double* eta, const double* S0, const double* M0,
                          const double* dO, const double* dST, const double* dMT, double* dq,
                          double* dk, double* dv, double* dalpha, double* dbeta, double* dmu,
                          double* deta, double* dS0, double* dM0, int b, int h, int T, int H,
                          int Dk, int Dv, int col_block, double* Ss, double* Ms, double* vts,
                          double* Sh, double* Mh, double* P, double* dvt)
{
    for (int t = 0; t < T; ++t) {
        const size_t g = IDX_GATE(b, t, h, T, H);
        dalpha[g] = 0.0;
        dmu[g] = 0.0;
        deta[g] = 0.0;
        if (dbeta) dbeta[g] = 0.0;
        for (int i = 0; i < Dk; ++i) {
            dq[IDX_TOK(b, t, h, i, T, H, Dk)] = 0.0;
            dk[IDX_TOK(b, t, h, i, T, H, Dk)] = 0.0;
        }
    }
    for (int c0 = 0; c0 < Dv; c0 += col_block) {
        const int nc = (c0 + col_block <= Dv) ? col_block : Dv - c0;
        const size_t st = (size_t)Dk * nc;   /* one stored state */
        /* forward, keeping S_t, M_t for t = 0..T and vt_t */
        for (int i = 0; i < Dk; ++i)
            for (int c = 0; c < nc; ++c) {
                Ss[(size_t)i * nc + c] = S0 ? S0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;
                Ms[(size_t)i * nc + c] = M0 ? M0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;
            }
        for (int t = 0; t < T; ++t) {
            const size_t g = IDX_GATE(b, t, h, T, H);
            const double a = alpha[g], m = mu[g], e = eta[g], s = beta ? beta[g] : 1.0;
            const double* kt = k + IDX_TOK(b, t, h, 0, T, H, Dk);
            double* Sn = Ss + st * (t + 1);
            double* Mn = Ms + st * (t + 1);
            memcpy(Sn, Ss + st * t, sizeof(double) * st);
            memcpy(Mn, Ms + st * t, sizeof(double) * st);
            token_step(kt, v + IDX_TOK(b, t, h, c0, T, H, Dv), a, m, e, s, Sn, Mn,
                       vts + (size_t)nc * t, Dk, nc);
        }
        /* backward, last token first */
        for (int i = 0; i < Dk; ++i)
            for (int c = 0; c < nc; ++c) {
                Sh[(size_t)i * nc + c] = dST ? dST[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;
                Mh[(size_t)i * nc + c] = dMT ? dMT[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] : 0.0;
            }
        for (int t = T - 1; t >= 0; --t) {
            const size_t g = IDX_GATE(b, t, h, T, H);
            const double a = alpha[g], m = mu[g], e = eta[g], s = beta ? beta[g] : 1.0;
            const double* kt = k + IDX_TOK(b, t, h, 0, T, H, Dk);
            const double* qt = q + IDX_TOK(b, t, h, 0, T, H, Dk);
            const double* dot = dO + IDX_TOK(b, t, h, c0, T, H, Dv);
            const double* Sp = Ss + st * t;         /* S_{t-1} */
            const double* Mp = Ms + st * t;         /* M_{t-1} */
            const double* Sn = Ss + st * (t + 1);   /* S_t */
            const double* Mn = Ms + st * (t + 1);   /* M_t */
            const double* vt = vts + (size_t)nc * t;
            double* dqt = dq + IDX_TOK(b, t, h, 0, T, H, Dk);
            double* dkt = dk + IDX_TOK(b, t, h, 0, T, H, Dk);
            double* dvv = dv + IDX_TOK(b, t, h, c0, T, H, Dv);
            double ga = 0.0, gb = 0.0, gm = 0.0, ge = 0.0;
            /* read-out */
            for (int i = 0; i < Dk; ++i) {
                double acc = 0.0;
                for (int c = 0; c < nc; ++c) {
                    const size_t x = (size_t)i * nc + c;
                    Sh[x] += qt[i] * dot[c];
                    acc += Sn[x] * dot[c];
                }
                dqt[i] += acc;
            }
            /* memory step */
            for (size_t x = 0; x < st; ++x) {
                ga += Sp[x] * Sh[x];
                gb -= Mn[x] * Sh[x];
                P[x] = Mh[x] - s * Sh[x];
            }
            /* momentum step */
            for (int c = 0; c < nc; ++c) dvt[c] = 0.0;
            for (int i = 0; i < Dk; ++i) {
                double acc = 0.0;
                for (int c = 0; c < nc; ++c) {
                    const size_t x = (size_t)i * nc + c;
                    gm += Mp[x] * P[x];
                    acc += P[x] * vt[c];
                    dvt[c] += P[x] * kt[i];
                }
                ge -= kt[i] * acc;
                dkt[i] -= e * acc;
            }
            for (int c = 0; c < nc; ++c) dvt[c] *= -e;
            /* residual */
            for (int c = 0; c < nc; ++c) dvv[c] = dvt[c];
            for (int i = 0; i < Dk; ++i) {
                double acc = 0.0;
                for (int c = 0; c < nc; ++c) acc += Sp[(size_t)i * nc + c] * dvt[c];
                dkt[i] -= a * acc;
                ga -= kt[i] * acc;
            }
            /* hand on to token t-1 */
            for (int i = 0; i < Dk; ++i)
                for (int c = 0; c < nc; ++c) {
                    const size_t x = (size_t)i * nc + c;
                    Sh[x] = a * Sh[x] - a * kt[i] * dvt[c];
                    Mh[x] = m * P[x];
                }
            dalpha[g] += ga;
            dmu[g] += gm;
            deta[g] += ge;
            if (dbeta) dbeta[g] += gb;
        }
        for (int i = 0; i < Dk; ++i)
            for (int c = 0; c < nc; ++c) {
                if (dS0) dS0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] = Sh[(size_t)i * nc + c];
                if (dM0) dM0[IDX_STATE(b, h, i, c0 + c, H, Dk, Dv)] = Mh[(size_t)i * nc + c];
            }
    }
}

/*
 * Gradients of a loss L through the recurrence, given dO [B,T,H,Dv] and
 * optional dST, dMT [B,H,Dk,Dv] (NULL: zero).  Outputs: dq, dk [B,T,H,Dk];
 * dv [B,T,H,Dv]; dalpha, dmu, deta [B,T,H]; dbeta [B,T,H] or NULL (then
 * not computed); dS0, dM0 [B,H,Dk,Dv] or NULL.  beta NULL means beta = 1.
 * Memory: 2 (T + 1) Dk col_block doubles per thread.  Returns 0 on success.
 */
int mdn_oracle_recurrence_backward(const double* q, const double* k, const double* v,
                                   const double* alpha, const double* beta, const double* mu,
                                   const double* eta, const double* S0, const double* M0,
                                   const double* dO, const double* dST, const double* dMT,
                                   double* dq, double* dk, double* dv, double* dalpha,
                                   double* dbeta, double* dmu, double* deta, double* dS0,
                                   double* dM0, int B, int T, int H, int Dk, int Dv,
                                   int col_block, int nthreads)
{
    if (!q || !k || !v || !alpha || !mu || !eta || !dO) return 1;
    if (!dq || !dk || !dv || !dalpha || !dmu || !deta) return 1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return 2;
    if (col_block <= 0 || col_block > Dv) col_block = Dv;
    const long units = (long)B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : failed)
    {
        const size_t st = (size_t)Dk * col_block;
        double* Ss = (double*)malloc(sizeof(double) * st * ((size_t)T + 1));
        double* Ms = (double*)malloc(sizeof(double) * st * ((size_t)T + 1));
        double* vts = (double*)malloc(sizeof(double) * (size_t)col_block * (T > 0 ? T : 1));
        double* Sh = (double*)malloc(sizeof(double) * st);
        double* Mh = (double*)malloc(sizeof(double) * st);
        double* P = (double*)malloc(sizeof(double) * st);
        double* dvt = (double*)malloc(sizeof(double) * (size_t)col_block);
        const int ok = Ss && Ms && vts && Sh && Mh && P && dvt;
        if (!ok) failed = 1;
#pragma omp for schedule(dynamic, 1)
        for (long u = 0; u < units; ++u) {
            if (!ok) continue;
            const int h = (int)(u % H);
            const int b = (int)(u / H);
            backward_unit(q, k, v, alpha, beta, mu, eta, S0, M0, dO, dST, dMT, dq, dk, dv,
                          dalpha, dbeta, dmu, deta, dS0, dM0, b, h, T, H, Dk, Dv, col_block,
                          Ss, Ms, vts, Sh, Mh, P, dvt);
        }
        free(Ss);
        free(Ms);
        free(vts);
        free(Sh);
        free(Mh);
        free(P);
        free(dvt);
    }
    return failed ? 3 : 0;
}

/* ------------------------------------------------------------------------ */
/* Brute-force chunkwise evaluator (tiny inputs only)                        */
/* ------------------------------------------------------------------------ */

/*
 * Variant flags.  0 is the consistent reading of the pages; each other flag
 * switches in one of the readings the pages themselves flag as erroneous, so
 * that tests can show they break parity:
 *   BF_UNSHIFTED_MASK  the residual system uses Gamma with its diagonal
 *                      deleted instead of Gamma shifted down one row
 *                      ([MDN slides] backup "a one-row shift is essential").
 *   BF_EQ8_TYPO        carry write term Diag(gamma_CC / gamma_C,:) instead of
 *                      Diag(Gamma_C,:) ([MDN notes] Sec. 2.3, last paragraph).
 *   BF_EQ10_TYPO       b_i = mubar_i * c_i (cumulative log mu) instead of
 *                      abar_i * c_i ([MDN slides] backup "use the consistent
 *                      log-domain coefficients").
 * Gamma forms (gamma_form):
 *   0  product-sum definition  sum_{r=j}^{i} beta_r prod_{u=r+1}^{i} alpha_u
 *      prod_{u=j+1}^{r} mu_u   ([MDN notes] Sec. 2.3)
 *   1  cumulative ratio (abar_i / mubar_j)(c_i - c_{j-1})   ([MDN slides] Eqs. (7)-(9))
 *   2  log domain exp(A_i + l_i - U_j)[1 - exp(l_{j-1} - l_i)]
 *      ([MDN slides] backup on log-domain coefficients; [MDN notes] Sec. 2.6)
 *   Forms 1 and 2 divide by mubar and therefore need mu > 0.
 */
#define BF_UNSHIFTED_MASK 1
#define BF_EQ8_TYPO 2
#define BF_EQ10_TYPO 4

/* Gamma (n x n, lower with diagonal, zero above) for one chunk, 1-based
 * gates a[1..n], m[1..n], s[1..n] stored at a[0..n-1]. */
static void chunk_gamma(int n, const double* a, const double* m, const double* s, int form,
                        double* G)
{
    memset(G, 0, sizeof(double) * (size_t)n * n);
    if (form == 0) {
        for (int i = 0; i < n; ++i)
            for (int j = 0; j <= i; ++j) {
                double acc = 0.0;
                for (int r = j; r <= i; ++r) {
                    double pa = 1.0, pm = 1.0;
                    for (int u = r + 1; u <= i; ++u) pa *= a[u];
                    for (int u = j + 1; u <= r; ++u) pm *= m[u];
                    acc += s[r] * pa * pm;
                }
                G[(size_t)i * n + j] = acc;
            }
        return;
    }
    /* cumulative products and c (index 0 of abar/mbar/cc means "before the
     * chunk": abar_0 = mubar_0 = 1, c_0 = 0) */
    double* abar = (double*)malloc(sizeof(double) * (n + 1));
    double* mbar = (double*)malloc(sizeof(double) * (n + 1));
    double* cc = (double*)malloc(sizeof(double) * (n + 1));
    abar[0] = mbar[0] = 1.0;
    cc[0] = 0.0;
    for (int i = 1; i <= n; ++i) {
        abar[i] = abar[i - 1] * a[i - 1];
        mbar[i] = mbar[i - 1] * m[i - 1];
        cc[i] = cc[i - 1] + s[i - 1] * mbar[i] / abar[i];
    }
    if (form == 1) {
        for (int i = 1; i <= n; ++i)
            for (int j = 1; j <= i; ++j)
                G[(size_t)(i - 1) * n + (j - 1)] = abar[i] / mbar[j] * (cc[i] - cc[j - 1]);
    } else {
        /* A_i = sum log alpha, U_i = sum log mu, l_i = log c_i computed as a
         * log-sum-exp of log beta_r + U_r - A_r; l_0 = -inf. */
        double* A = (double*)malloc(sizeof(double) * (n + 1));
        double* U = (double*)malloc(sizeof(double) * (n + 1));
        double* l = (double*)malloc(sizeof(double) * (n + 1));
        A[0] = U[0] = 0.0;
        l[0] = -INFINITY;
        for (int i = 1; i <= n; ++i) {
            A[i] = A[i - 1] + log(a[i - 1]);
            U[i] = U[i - 1] + log(m[i - 1]);
            /* stable prefix log-sum-exp over r <= i: subtract the max */
            double mx = -INFINITY;
            for (int r = 1; r <= i; ++r) {
                const double x = log(s[r - 1]) + U[r] - A[r];
                if (x > mx) mx = x;
            }
            double acc = 0.0;
            for (int r = 1; r <= i; ++r) acc += exp(log(s[r - 1]) + U[r] - A[r] - mx);
            l[i] = mx + log(acc);
        }
        for (int i = 1; i <= n; ++i)
            for (int j = 1; j <= i; ++j)
                G[(size_t)(i - 1) * n + (j - 1)] =
                    exp(A[i] + l[i] - U[j]) * (1.0 - exp(l[j - 1] - l[i]));
        free(A);
        free(U);
        free(l);
    }
    free(abar);
    free(mbar);
    free(cc);
}

/* Dense inverse by Gauss-Jordan elimination with partial pivoting (n x n,
 * row-major).  Returns nonzero if singular. */
static int gauss_jordan_inverse(int n, const double* Ain, double* Inv)
{
    const int w = 2 * n;
    double* W = (double*)calloc((size_t)n * w, sizeof(double));
    if (!W) return 1;
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < n; ++j) W[(size_t)i * w + j] = Ain[(size_t)i * n + j];
        W[(size_t)i * w + n + i] = 1.0;
    }
    for (int col = 0; col < n; ++col) {
        int piv = col;
        for (int r = col + 1; r < n; ++r)
            if (fabs(W[(size_t)r * w + col]) > fabs(W[(size_t)piv * w + col])) piv = r;
        if (W[(size_t)piv * w + col] == 0.0) {
            free(W);
            return 2;
        }
        if (piv != col)
            for (int j = 0; j < w; ++j) {
                const double t = W[(size_t)col * w + j];
                W[(size_t)col * w + j] = W[(size_t)piv * w + j];
                W[(size_t)piv * w + j] = t;
            }
        const double d = W[(size_t)col * w + col];
        for (int j = 0; j < w; ++j) W[(size_t)col * w + j] /= d;
        for (int r = 0; r < n; ++r) {
            if (r == col) continue;
            const double f = W[(size_t)r * w + col];
            if (f == 0.0) continue;
            for (int j = 0; j < w; ++j) W[(size_t)r * w + j] -= f * W[(size_t)col * w + j];
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) Inv[(size_t)i * n + j] = W[(size_t)i * w + n + j];
    free(W);
    return 0;
}

/*
 * Chunkwise evaluation of one (b, h), chunk length C (the last chunk may be
 * shorter: it then has n = T - (N_c - 1) C rows and the carry uses its row n).
 * Everything follows the page statements literally, in matrix form:
 *   Sec. 2.3  abar, mubar, c, b = abar*c, Gamma                (Eqs. (7)-(9))
 *   Sec. 2.4  [I + (P Khat^T) o Gamma^-] Vt = V - Diag(abar^-) P S0
 *                                              + Diag(b^-) P M0  (Eqs. (15)-(18))
 *             T = inverse, U = T V, Y = T Diag(abar^-) P, Z = T Diag(b^-) P,
 *             Vt = U - Y S0 + Z M0
 *   Sec. 2.5  O = Diag(abar) Q S0 - Diag(b) Q M0 + [(Q Khat^T) o Gamma] Vt
 *             S_next = abar_C S0 - b_C M0 + [Diag(Gamma_C,:) Khat]^T Vt
 *             M_next = mubar_C M0 - [Diag(mubar_C / mubar) Khat]^T Vt
 *                                                           (Eqs. (40)-(42))
 * with P = Diag(alpha) K, Khat = Diag(eta) K.  mubar_C / mubar_j is formed as
 * the product of mu over (j, C], its definition, so that mu = 0 is allowed.
 */
static int chunk_bruteforce_head(const double* q, const double* k, const double* v,
                                 const double* alpha, const double* beta, const double* mu,
                                 const double* eta, const double* S0, const double* M0,
                                 double* O, double* ST, double* MT, int b, int h, int T, int H,
                                 int Dk, int Dv, int C, int gamma_form, int flags)
{
    double* S = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
    double* M = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
    double* Sn = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
    double* Mn = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
    double* G = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Gm = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* L = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Tm = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Pm = (double*)malloc(sizeof(double) * (size_t)C * Dk);
    double* Kh = (double*)malloc(sizeof(double) * (size_t)C * Dk);
    double* Qm = (double*)malloc(sizeof(double) * (size_t)C * Dk);
    double* Vm = (double*)malloc(sizeof(double) * (size_t)C * Dv);
    double* U = (double*)malloc(sizeof(double) * (size_t)C * Dv);
    double* Y = (double*)malloc(sizeof(double) * (size_t)C * Dk);
    double* Z = (double*)malloc(sizeof(double) * (size_t)C * Dk);
    double* Vt = (double*)malloc(sizeof(double) * (size_t)C * Dv);
    double* a = (double*)malloc(sizeof(double) * C);
    double* m = (double*)malloc(sizeof(double) * C);
    double* e = (double*)malloc(sizeof(double) * C);
    double* s = (double*)malloc(sizeof(double) * C);
    double* abar = (double*)malloc(sizeof(double) * (C + 1));
    double* mbar = (double*)malloc(sizeof(double) * (C + 1));
    double* cc = (double*)malloc(sizeof(double) * (C + 1));
    double* bb = (double*)malloc(sizeof(double) * (C + 1));
    int rc = 0;
    if (!S || !M || !Sn || !Mn || !G || !Gm || !L || !Tm || !Pm || !Kh || !Qm || !Vm || !U ||
        !Y || !Z || !Vt || !a || !m || !e || !s || !abar || !mbar || !cc || !bb) {
        rc = 3;
        goto done;
    }
    for (int i = 0; i < Dk; ++i)
        for (int c = 0; c < Dv; ++c) {
            S[(size_t)i * Dv + c] = S0 ? S0[IDX_STATE(b, h, i, c, H, Dk, Dv)] : 0.0;
            M[(size_t)i * Dv + c] = M0 ? M0[IDX_STATE(b, h, i, c, H, Dk, Dv)] : 0.0;
        }

    for (int t0 = 0; t0 < T; t0 += C) {
        const int n = (t0 + C <= T) ? C : T - t0;
        for (int i = 0; i < n; ++i) {
            const size_t g = IDX_GATE(b, t0 + i, h, T, H);
            a[i] = alpha[g];
            m[i] = mu[g];
            e[i] = eta[g];
            s[i] = beta ? beta[g] : 1.0;
            for (int d = 0; d < Dk; ++d) {
                const double kk = k[IDX_TOK(b, t0 + i, h, d, T, H, Dk)];
                Pm[(size_t)i * Dk + d] = a[i] * kk;
                Kh[(size_t)i * Dk + d] = e[i] * kk;
                Qm[(size_t)i * Dk + d] = q[IDX_TOK(b, t0 + i, h, d, T, H, Dk)];
            }
            for (int c = 0; c < Dv; ++c) Vm[(size_t)i * Dv + c] = v[IDX_TOK(b, t0 + i, h, c, T, H, Dv)];
        }
        /* scalar coefficients; index 0 = before the chunk */
        abar[0] = mbar[0] = 1.0;
        cc[0] = bb[0] = 0.0;
        for (int i = 1; i <= n; ++i) {
            abar[i] = abar[i - 1] * a[i - 1];
            mbar[i] = mbar[i - 1] * m[i - 1];
        }
        /* c_i = sum_{r<=i} beta_r mubar_r / abar_r and b_i = abar_i c_i; b is
         * formed from its expansion sum_{r<=i} beta_r mubar_r prod_{u=r+1}^{i}
         * alpha_u so that no division is needed. */
        for (int i = 1; i <= n; ++i) {
            double acc = 0.0;
            for (int r = 1; r <= i; ++r) {
                double pa = 1.0;
                for (int u = r + 1; u <= i; ++u) pa *= a[u - 1];
                acc += s[r - 1] * mbar[r] * pa;
            }
            bb[i] = acc;
            if (flags & BF_EQ10_TYPO) {
                /* mubar_i * c_i = mubar_i / abar_i * b_i */
                bb[i] = mbar[i] / abar[i] * acc;
            }
        }
        chunk_gamma(n, a, m, s, gamma_form, G);
        /* Gamma^- : Gamma shifted down one row (or the flagged wrong mask) */
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                double x = 0.0;
                if (flags & BF_UNSHIFTED_MASK) {
                    if (j < i) x = G[(size_t)i * n + j];
                } else {
                    if (j < i) x = G[(size_t)(i - 1) * n + j];
                }
                Gm[(size_t)i * n + j] = x;
            }
        /* L = I + (P Khat^T) o Gamma^- */
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                double pk = 0.0;
                for (int d = 0; d < Dk; ++d) pk += Pm[(size_t)i * Dk + d] * Kh[(size_t)j * Dk + d];
                L[(size_t)i * n + j] = (i == j ? 1.0 : 0.0) + pk * Gm[(size_t)i * n + j];
            }
        if (gauss_jordan_inverse(n, L, Tm)) {
            rc = 4;
            goto done;
        }
        /* U = T V ; Y = T Diag(abar^-) P ; Z = T Diag(b^-) P
         * abar^- = (1, abar_1, ..., abar_{n-1}), b^- = (0, b_1, ..., b_{n-1}) */
        for (int i = 0; i < n; ++i) {
            for (int c = 0; c < Dv; ++c) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += Tm[(size_t)i * n + j] * Vm[(size_t)j * Dv + c];
                U[(size_t)i * Dv + c] = acc;
            }
            for (int d = 0; d < Dk; ++d) {
                double ay = 0.0, az = 0.0;
                for (int j = 0; j < n; ++j) {
                    ay += Tm[(size_t)i * n + j] * abar[j] * Pm[(size_t)j * Dk + d];
                    az += Tm[(size_t)i * n + j] * bb[j] * Pm[(size_t)j * Dk + d];
                }
                Y[(size_t)i * Dk + d] = ay;
                Z[(size_t)i * Dk + d] = az;
            }
        }
        /* Vt = U - Y S0 + Z M0 */
        for (int i = 0; i < n; ++i)
            for (int c = 0; c < Dv; ++c) {
                double acc = U[(size_t)i * Dv + c];
                for (int d = 0; d < Dk; ++d)
                    acc += -Y[(size_t)i * Dk + d] * S[(size_t)d * Dv + c] +
                           Z[(size_t)i * Dk + d] * M[(size_t)d * Dv + c];
                Vt[(size_t)i * Dv + c] = acc;
            }
        /* O = Diag(abar) Q S0 - Diag(b) Q M0 + [(Q Khat^T) o Gamma] Vt */
        for (int i = 0; i < n; ++i) {
            for (int j = 0; j < n; ++j) {
                double qk = 0.0;
                for (int d = 0; d < Dk; ++d) qk += Qm[(size_t)i * Dk + d] * Kh[(size_t)j * Dk + d];
                Gm[(size_t)i * n + j] = (j <= i) ? qk * G[(size_t)i * n + j] : 0.0;
            }
            for (int c = 0; c < Dv; ++c) {
                double acc = 0.0;
                for (int d = 0; d < Dk; ++d)
                    acc += abar[i + 1] * Qm[(size_t)i * Dk + d] * S[(size_t)d * Dv + c] -
                           bb[i + 1] * Qm[(size_t)i * Dk + d] * M[(size_t)d * Dv + c];
                for (int j = 0; j < n; ++j) acc += Gm[(size_t)i * n + j] * Vt[(size_t)j * Dv + c];
                O[IDX_TOK(b, t0 + i, h, c, T, H, Dv)] = acc;
            }
        }
        /* carry: S_next, M_next from the OLD S0, M0 */
        for (int d = 0; d < Dk; ++d)
            for (int c = 0; c < Dv; ++c) {
                double ws = 0.0, wm = 0.0;
                for (int j = 0; j < n; ++j) {
                    double gs = G[(size_t)(n - 1) * n + j];
                    if (flags & BF_EQ8_TYPO) gs = G[(size_t)(n - 1) * n + (n - 1)] / gs;
                    double ratio = 1.0; /* mubar_n / mubar_{j+1} = prod mu over (j+1, n] */
                    for (int u = j + 1; u < n; ++u) ratio *= m[u];
                    ws += gs * Kh[(size_t)j * Dk + d] * Vt[(size_t)j * Dv + c];
                    wm += ratio * Kh[(size_t)j * Dk + d] * Vt[(size_t)j * Dv + c];
                }
                const size_t x = (size_t)d * Dv + c;
                Sn[x] = abar[n] * S[x] - bb[n] * M[x] + ws;
                Mn[x] = mbar[n] * M[x] - wm;
            }
        memcpy(S, Sn, sizeof(double) * (size_t)Dk * Dv);
        memcpy(M, Mn, sizeof(double) * (size_t)Dk * Dv);
    }
    for (int i = 0; i < Dk; ++i)
        for (int c = 0; c < Dv; ++c) {
            if (ST) ST[IDX_STATE(b, h, i, c, H, Dk, Dv)] = S[(size_t)i * Dv + c];
            if (MT) MT[IDX_STATE(b, h, i, c, H, Dk, Dv)] = M[(size_t)i * Dv + c];
        }
done:
    free(S); free(M); free(Sn); free(Mn); free(G); free(Gm); free(L); free(Tm);
    free(Pm); free(Kh); free(Qm); free(Vm); free(U); free(Y); free(Z); free(Vt);
    free(a); free(m); free(e); free(s); free(abar); free(mbar); free(cc); free(bb);
    return rc;
}

int mdn_oracle_chunk_bruteforce(const double* q, const double* k, const double* v,
                                const double* alpha, const double* beta, const double* mu,
                                const double* eta, const double* S0, const double* M0,
                                double* O, double* ST, double* MT, int B, int T, int H, int Dk,
                                int Dv, int C, int gamma_form, int flags)
{
    if (!q || !k || !v || !alpha || !mu || !eta || !O) return 1;
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0 || C <= 0) return 2;
    if (gamma_form < 0 || gamma_form > 2) return 2;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int rc = chunk_bruteforce_head(q, k, v, alpha, beta, mu, eta, S0, M0, O, ST,
                                                 MT, b, h, T, H, Dk, Dv, C, gamma_form, flags);
            if (rc) return rc;
        }
    return 0;
}

/* Gamma of one chunk in a chosen form, exposed so tests can compare the
 * three statements of gamma directly.  n x n row-major output. */
int mdn_oracle_chunk_gamma(const double* alpha, const double* beta, const double* mu, int n,
                           int form, double* G)
{
    if (!alpha || !mu || !G || n <= 0 || form < 0 || form > 2) return 1;
    double* s = (double*)malloc(sizeof(double) * n);
    if (!s) return 3;
    for (int i = 0; i < n; ++i) s[i] = beta ? beta[i] : 1.0;
    chunk_gamma(n, alpha, mu, s, form, G);
    free(s);
    return 0;
}
