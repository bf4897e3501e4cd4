"""Pins for the fp64 oracle: results fixed by the pages and by mathematics,
each computed here WITHOUT the oracle's own formula, so that a dropped term,
a wrong sign or index or a transposed operand in the oracle fails one of them.

Every pin takes the loaded oracle library (``lib``) so the same checks can be
run against deliberately broken builds of the oracle (see
``test_oracle_mutants.py``).  Each raises AssertionError when violated.

Sources:
  [MDN slides]  "MDN: Parallelizing Stepwise Momentum for Delta Linear Attention"
  [MDN notes]   reading notes on the same paper
  [PDN slides]  "Preconditioned DeltaNet" (DeltaNet update and its two-key
                chunk algorithm)
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = 1e-12


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return float(np.max(np.abs(a - b))) / scale if a.size else 0.0


def _unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _gates(rng, shape, lo_a=0.5, hi_a=1.0, lo_m=0.0, hi_m=0.9, lo_e=0.05, hi_e=1.0):
    return (rng.uniform(lo_a, hi_a, shape), rng.uniform(lo_m, hi_m, shape),
            rng.uniform(lo_e, hi_e, shape))


# --------------------------------------------------------------------------
# P1: one token, closed form ([MDN slides] Sec. 3.1 Eqs. (3)-(5) at T = 1)
# --------------------------------------------------------------------------
def pin_one_token(lib):
    """T = 1 from arbitrary S0, M0 (and an explicit beta):
        vt  = v - alpha S0^T k
        S_1 = alpha S0 - beta mu M0 + beta eta k vt^T
        M_1 = mu M0 - eta k vt^T,   o = S_1^T q
    and, from zero state, o = beta eta (q . k) v."""
    rng = np.random.default_rng(11)
    B, H, Dk, Dv = 2, 3, 5, 4
    q = rng.standard_normal((B, 1, H, Dk))
    k = rng.standard_normal((B, 1, H, Dk))
    v = rng.standard_normal((B, 1, H, Dv))
    a, m, e = _gates(rng, (B, 1, H))
    s = rng.uniform(0.2, 1.0, (B, 1, H))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    M0 = rng.standard_normal((B, H, Dk, Dv))
    for beta in (None, s):
        O, ST, MT = oracle.recurrence(q, k, v, a, m, e, beta, S0, M0, lib=lib)
        bb = np.ones_like(a) if beta is None else beta
        for b_ in range(B):
            for h in range(H):
                al, mu, et, be = a[b_, 0, h], m[b_, 0, h], e[b_, 0, h], bb[b_, 0, h]
                kk, qq, vv = k[b_, 0, h], q[b_, 0, h], v[b_, 0, h]
                vt = vv - al * (S0[b_, h].T @ kk)
                S1 = al * S0[b_, h] - be * mu * M0[b_, h] + be * et * np.outer(kk, vt)
                M1 = mu * M0[b_, h] - et * np.outer(kk, vt)
                assert _rel(ST[b_, h], S1) < TOL
                assert _rel(MT[b_, h], M1) < TOL
                assert _rel(O[b_, 0, h], S1.T @ qq) < TOL
    # zero initial state: o = eta (q.k) v  (beta == 1)
    O, _, _ = oracle.recurrence(q, k, v, a, m, e, lib=lib)
    expect = (e[..., None] * np.sum(q * k, axis=-1, keepdims=True)) * v
    assert _rel(O, expect) < TOL


# --------------------------------------------------------------------------
# P2: two tokens, the two propagation paths ([MDN slides] "One error can affect
# several future writes"; [MDN notes] Sec. 2.2 two-step example)
# --------------------------------------------------------------------------
def pin_residuals(lib):
    """The residual the recurrence reports is vt_t = v_t - alpha_t S_{t-1}^T k_t
    ([MDN slides] Sec. 3.1 Eq. (3)): at T = 1 from arbitrary S0 it is the
    closed form; at T = 2 the second one is taken against S_1, rebuilt from
    the first residual as S_1 = alpha_1 S0 - beta_1 (mu_1 M0 - eta_1 k_1 vt_1^T)."""
    rng = np.random.default_rng(12)
    B, H, Dk, Dv = 1, 2, 4, 3
    q = rng.standard_normal((B, 2, H, Dk))
    k = rng.standard_normal((B, 2, H, Dk))
    v = rng.standard_normal((B, 2, H, Dv))
    a, m, e = _gates(rng, (B, 2, H))
    s = rng.uniform(0.2, 1.0, (B, 2, H))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    M0 = rng.standard_normal((B, H, Dk, Dv))
    _, _, _, VT = oracle.recurrence(q, k, v, a, m, e, s, S0, M0, lib=lib, return_vt=True)
    for h in range(H):
        vt1 = v[0, 0, h] - a[0, 0, h] * S0[0, h].T @ k[0, 0, h]
        assert _rel(VT[0, 0, h], vt1) < TOL
        M1 = m[0, 0, h] * M0[0, h] - e[0, 0, h] * np.outer(k[0, 0, h], vt1)
        S1 = a[0, 0, h] * S0[0, h] - s[0, 0, h] * M1
        assert _rel(VT[0, 1, h], v[0, 1, h] - a[0, 1, h] * S1.T @ k[0, 1, h]) < TOL


def pin_two_tokens(lib):
    """From zero state, the first residual reaches S_2 with weight
    (alpha_2 beta_1 + beta_2 mu_2):
        S_2 = (alpha_2 beta_1 + beta_2 mu_2) eta_1 k_1 v_1^T + beta_2 eta_2 k_2 vt_2^T
        vt_2 = v_2 - alpha_2 beta_1 eta_1 (k_1 . k_2) v_1
        M_2 = -mu_2 eta_1 k_1 v_1^T - eta_2 k_2 vt_2^T."""
    rng = np.random.default_rng(12)
    B, H, Dk, Dv = 1, 4, 6, 3
    q = rng.standard_normal((B, 2, H, Dk))
    k = rng.standard_normal((B, 2, H, Dk))
    v = rng.standard_normal((B, 2, H, Dv))
    a, m, e = _gates(rng, (B, 2, H))
    s = rng.uniform(0.2, 1.0, (B, 2, H))
    for beta in (None, s):
        O, ST, MT = oracle.recurrence(q, k, v, a, m, e, beta, lib=lib)
        bb = np.ones_like(a) if beta is None else beta
        for h in range(H):
            k1, k2 = k[0, 0, h], k[0, 1, h]
            v1, v2 = v[0, 0, h], v[0, 1, h]
            a2, m2 = a[0, 1, h], m[0, 1, h]
            e1, e2 = e[0, 0, h], e[0, 1, h]
            b1, b2 = bb[0, 0, h], bb[0, 1, h]
            vt2 = v2 - a2 * b1 * e1 * np.dot(k1, k2) * v1
            S2 = (a2 * b1 + b2 * m2) * e1 * np.outer(k1, v1) + b2 * e2 * np.outer(k2, vt2)
            M2 = -m2 * e1 * np.outer(k1, v1) - e2 * np.outer(k2, vt2)
            S1 = b1 * e1 * np.outer(k1, v1)
            assert _rel(ST[0, h], S2) < TOL
            assert _rel(MT[0, h], M2) < TOL
            assert _rel(O[0, 0, h], S1.T @ q[0, 0, h]) < TOL
            assert _rel(O[0, 1, h], S2.T @ q[0, 1, h]) < TOL


# --------------------------------------------------------------------------
# P3: mu = 0 gives the gated delta rule; alpha = 1 then gives DeltaNet
# ([MDN slides] Eqs. (3)-(5) note; [MDN notes] Sec. 2.2; [PDN slides]
# "DeltaNet already corrects errors")
# --------------------------------------------------------------------------
def _gdn_loop(q, k, v, a, e, S0=None):
    """Independent single-state loop S = aS + e k (v - a S^T k)^T, o = S^T q."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    O = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    for b_ in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else S0[b_, h].copy()
            for t in range(T):
                kk = k[b_, t, h]
                S = a[b_, t, h] * S + e[b_, t, h] * np.outer(kk, v[b_, t, h] - a[b_, t, h] * S.T @ kk)
                O[b_, t, h] = S.T @ q[b_, t, h]
            ST[b_, h] = S
    return O, ST


def _deltanet_loop(q, k, v, beta, S0=None):
    """DeltaNet in the [PDN slides] orientation: S in R^{dv x dk},
    S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T, o_t = S_t q_t."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    O = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dv, Dk))
    for b_ in range(B):
        for h in range(H):
            S = np.zeros((Dv, Dk)) if S0 is None else S0[b_, h].T.copy()
            for t in range(T):
                kk = k[b_, t, h]
                S = S + beta[b_, t, h] * np.outer(v[b_, t, h] - S @ kk, kk)
                O[b_, t, h] = S @ q[b_, t, h]
            ST[b_, h] = S
    return O, ST


def pin_gdn_reduction(lib):
    rng = np.random.default_rng(13)
    B, T, H, Dk, Dv = 2, 19, 2, 7, 5
    q = rng.standard_normal((B, T, H, Dk))
    k = _unit_rows(rng, (B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    a, _, e = _gates(rng, (B, T, H))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    zero = np.zeros_like(a)
    O, ST, MT = oracle.recurrence(q, k, v, a, zero, e, None, S0, None, lib=lib)
    Og, Sg = _gdn_loop(q, k, v, a, e, S0)
    assert _rel(O, Og) < TOL
    assert _rel(ST, Sg) < TOL
    # with mu = 0 the final momentum is the last write only: rank one,
    # M_T = -eta_T k_T vt_T^T with vt_T read from S_{T-1}
    _, S_prev, _ = oracle.recurrence(q[:, :-1], k[:, :-1], v[:, :-1], a[:, :-1], zero[:, :-1],
                                     e[:, :-1], None, S0, None, lib=lib)
    for b_ in range(B):
        for h in range(H):
            kk = k[b_, -1, h]
            vt = v[b_, -1, h] - a[b_, -1, h] * S_prev[b_, h].T @ kk
            assert _rel(MT[b_, h], -e[b_, -1, h] * np.outer(kk, vt)) < TOL
    # alpha = 1 as well: DeltaNet with write strength eta
    one = np.ones_like(a)
    O1, S1, _ = oracle.recurrence(q, k, v, one, zero, e, None, S0, None, lib=lib)
    Od, Sd = _deltanet_loop(q, k, v, e, S0)
    assert _rel(O1, Od) < TOL
    assert _rel(S1, np.swapaxes(Sd, -1, -2)) < TOL


# --------------------------------------------------------------------------
# P4: exact recall under the delta rule ([PDN slides] regression view;
# [MDN notes] Sec. 2.2: the update descends the key-value reconstruction loss)
# --------------------------------------------------------------------------
def pin_exact_recall(lib):
    """alpha = 1, mu = 0, eta = 1 and n <= d_k orthonormal keys: after writing
    (k_i, v_i), S^T k_i = v_i.  Reading with eta = 0 leaves S unchanged and
    returns v_i for q = k_i; overwriting k_j with v_j' changes only that
    association."""
    rng = np.random.default_rng(14)
    Dk, Dv, n = 8, 6, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:, :n].T                         # n orthonormal rows
    vals = rng.standard_normal((n, Dv))
    newv = rng.standard_normal(Dv)
    j = 2
    # tokens: n writes, n reads, one overwrite of key j, n reads
    ks = np.concatenate([keys, keys, keys[j:j + 1], keys])
    vs = np.concatenate([vals, np.zeros((n, Dv)), newv[None], np.zeros((n, Dv))])
    T = ks.shape[0]
    eta = np.concatenate([np.ones(n), np.zeros(n), np.ones(1), np.zeros(n)])
    q = ks.copy()
    shape = lambda x: x.reshape(1, T, 1, -1)
    O, ST, MT = oracle.recurrence(shape(q), shape(ks), shape(vs), np.ones((1, T, 1)),
                                  np.zeros((1, T, 1)), eta.reshape(1, T, 1), lib=lib)
    S = ST[0, 0]
    expect = vals.copy()
    expect[j] = newv
    assert _rel(S.T @ keys.T, expect.T) < 1e-12
    assert _rel(O[0, n:2 * n, 0], vals) < 1e-12           # reads before overwrite
    assert _rel(O[0, 2 * n + 1:, 0], expect) < 1e-12      # reads after overwrite
    # mu = 0 and a final read token (eta = 0): the momentum is exactly zero
    assert np.max(np.abs(MT)) == 0.0


# --------------------------------------------------------------------------
# P5: brute-force chunkwise equations vs the recurrence
# ([MDN slides] Eqs. (7)-(9), (15)-(18), (40)-(42) and backup frames;
# [MDN notes] Secs. 2.3-2.5: the chunk form is exact in real arithmetic)
# --------------------------------------------------------------------------
def _random_problem(rng, B, T, H, Dk, Dv, with_beta=False, state=True, mu_lo=0.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = _unit_rows(rng, (B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    a, m, e = _gates(rng, (B, T, H), lo_m=mu_lo)
    s = rng.uniform(0.2, 1.0, (B, T, H)) if with_beta else None
    S0 = rng.standard_normal((B, H, Dk, Dv)) if state else None
    M0 = rng.standard_normal((B, H, Dk, Dv)) if state else None
    return q, k, v, a, m, e, s, S0, M0


def pin_chunk_equations(lib):
    rng = np.random.default_rng(15)
    for C in (1, 2, 3, 5, 8, 64):
        for with_beta in (False, True):
            B, T, H, Dk, Dv = 1, 23, 2, 6, 5
            q, k, v, a, m, e, s, S0, M0 = _random_problem(rng, B, T, H, Dk, Dv, with_beta)
            Or, Sr, Mr = oracle.recurrence(q, k, v, a, m, e, s, S0, M0, lib=lib)
            Oc, Sc, Mc = oracle.chunk_bruteforce(q, k, v, a, m, e, s, S0, M0, chunk=C, lib=lib)
            assert _rel(Oc, Or) < 1e-11, (C, _rel(Oc, Or))
            assert _rel(Sc, Sr) < 1e-11
            assert _rel(Mc, Mr) < 1e-11
    # mu exactly zero in some tokens (the division-free statements allow it)
    q, k, v, a, m, e, s, S0, M0 = _random_problem(rng, 1, 17, 1, 4, 3)
    m[:, ::3] = 0.0
    Or, Sr, Mr = oracle.recurrence(q, k, v, a, m, e, None, S0, M0, lib=lib)
    Oc, Sc, Mc = oracle.chunk_bruteforce(q, k, v, a, m, e, None, S0, M0, chunk=8, lib=lib)
    assert _rel(Oc, Or) < 1e-11 and _rel(Sc, Sr) < 1e-11 and _rel(Mc, Mr) < 1e-11


def pin_gamma_forms_agree(lib):
    """The three statements of gamma (product sum, cumulative ratio, log
    domain) agree on tame inputs (mu >= 0.5, C <= 8)."""
    rng = np.random.default_rng(16)
    for n in (1, 2, 5, 8):
        a = rng.uniform(0.5, 1.0, n)
        m = rng.uniform(0.5, 0.95, n)
        s = rng.uniform(0.2, 1.0, n)
        g0 = oracle.chunk_gamma(a, m, s, form=0, lib=lib)
        g1 = oracle.chunk_gamma(a, m, s, form=1, lib=lib)
        g2 = oracle.chunk_gamma(a, m, s, form=2, lib=lib)
        assert _rel(g1, g0) < 1e-13 and _rel(g2, g0) < 1e-13
        # gamma_ii = beta_i: one write of the current residual
        assert _rel(np.diag(g0), s) < 1e-15
        # strictly upper part is zero (causal)
        assert np.all(np.triu(g0, 1) == 0)
    # chunk results with the ratio and log forms match the recurrence too
    q, k, v, a, m, e, s, S0, M0 = _random_problem(rng, 1, 13, 1, 5, 4, True, mu_lo=0.5)
    Or, Sr, Mr = oracle.recurrence(q, k, v, a, m, e, s, S0, M0, lib=lib)
    for form in (1, 2):
        Oc, Sc, Mc = oracle.chunk_bruteforce(q, k, v, a, m, e, s, S0, M0, chunk=5,
                                             gamma_form=form, lib=lib)
        assert _rel(Oc, Or) < 1e-11 and _rel(Sc, Sr) < 1e-11 and _rel(Mc, Mr) < 1e-11


def pin_flagged_readings_fail(lib):
    """The readings the pages flag as erroneous (unshifted mask, the Eq. (8)
    and Eq. (10) typos) must NOT reproduce the recurrence."""
    rng = np.random.default_rng(17)
    q, k, v, a, m, e, s, S0, M0 = _random_problem(rng, 1, 23, 1, 6, 5, True, mu_lo=0.3)
    Or, Sr, Mr = oracle.recurrence(q, k, v, a, m, e, s, S0, M0, lib=lib)
    for flag in (oracle.BF_UNSHIFTED_MASK, oracle.BF_EQ8_TYPO, oracle.BF_EQ10_TYPO):
        Oc, Sc, Mc = oracle.chunk_bruteforce(q, k, v, a, m, e, s, S0, M0, chunk=8, flags=flag,
                                             lib=lib)
        err = max(_rel(Oc, Or), _rel(Sc, Sr), _rel(Mc, Mr))
        assert err > 1e-3, (flag, err)


# --------------------------------------------------------------------------
# P6: frozen-step dynamics ([MDN slides] "Momentum permits damped oscillatory
# modes" and backup "the full spectrum includes orthogonal directions";
# [MDN notes] Sec. 2.7)
# --------------------------------------------------------------------------
def pin_frozen_step(lib):
    """Constant gates, one fixed unit key k, v = 0, S0 = k w^T + u z^T (u
    orthogonal to k), M0 = 0.  Then (k^T S_t, k^T M_t) = A^t e_1 w^T with
    A = [[alpha - alpha eta, -mu], [alpha eta, mu]] (trace alpha + mu -
    alpha eta, determinant alpha mu), and u^T S_t = alpha^t z^T."""
    rng = np.random.default_rng(18)
    Dk, Dv, T = 6, 4, 150
    for alpha, mu, eta in ((0.97, 0.8, 0.9), (0.9, 0.3, 0.5), (1.0, 0.95, 1.7)):
        kk = _unit_rows(rng, (Dk,))
        u = rng.standard_normal(Dk)
        u -= np.dot(u, kk) * kk
        u /= np.linalg.norm(u)
        w = rng.standard_normal(Dv)
        z = rng.standard_normal(Dv)
        S0 = (np.outer(kk, w) + np.outer(u, z)).reshape(1, 1, Dk, Dv)
        ks = np.broadcast_to(kk, (1, T, 1, Dk)).copy()
        g = lambda x: np.full((1, T, 1), x)
        O, ST, MT = oracle.recurrence(ks.copy(), ks, np.zeros((1, T, 1, Dv)), g(alpha), g(mu),
                                      g(eta), None, S0, None, lib=lib)
        A = np.array([[alpha - alpha * eta, -mu], [alpha * eta, mu]])
        x = np.linalg.matrix_power(A, T) @ np.array([1.0, 0.0])
        assert _rel(kk @ ST[0, 0], x[0] * w) < 1e-10
        assert _rel(kk @ MT[0, 0], x[1] * w) < 1e-10
        assert _rel(u @ ST[0, 0], alpha ** T * z) < 1e-10
        # read-out with q = k is k^T S_t at every step
        xt = np.array([1.0, 0.0])
        for t in range(T):
            xt = A @ xt
            assert _rel(O[0, t, 0], xt[0] * w) < 1e-10
        # eigenvalues: trace and determinant as stated
        lam = np.linalg.eigvals(A)
        assert abs(np.sum(lam) - (alpha + mu - alpha * eta)) < 1e-12
        assert abs(np.prod(lam) - alpha * mu) < 1e-12


# --------------------------------------------------------------------------
# P7: the second-order (momentum-eliminated) form ([MDN slides] backup
# "eliminating momentum reveals the second-order rule"; [MDN notes] Sec. 2.7)
# --------------------------------------------------------------------------
def pin_second_order(lib):
    """For t >= 2 (beta_{t-1} != 0):
    S_t = [(alpha_t + beta_t mu_t / beta_{t-1}) I - alpha_t beta_t eta_t k k^T] S_{t-1}
          - (beta_t mu_t alpha_{t-1} / beta_{t-1}) S_{t-2} + beta_t eta_t k_t v_t^T,
    S_1 from the one-step update.  Checked on every step's read-out."""
    rng = np.random.default_rng(19)
    B, T, H, Dk, Dv = 1, 31, 2, 5, 4
    q, k, v, a, m, e, s, S0, M0 = _random_problem(rng, B, T, H, Dk, Dv, with_beta=True)
    for beta in (None, s):
        O, ST, _ = oracle.recurrence(q, k, v, a, m, e, beta, S0, M0, lib=lib)
        bb = np.ones_like(a) if beta is None else beta
        for h in range(H):
            Sm2 = S0[0, h]
            k0 = k[0, 0, h]
            vt = v[0, 0, h] - a[0, 0, h] * Sm2.T @ k0
            Sm1 = a[0, 0, h] * Sm2 - bb[0, 0, h] * (m[0, 0, h] * M0[0, h]
                                                     - e[0, 0, h] * np.outer(k0, vt))
            assert _rel(O[0, 0, h], Sm1.T @ q[0, 0, h]) < 1e-11
            for t in range(1, T):
                kt = k[0, t, h]
                ratio = bb[0, t, h] * m[0, t, h] / bb[0, t - 1, h]
                St = ((a[0, t, h] + ratio) * Sm1
                      - a[0, t, h] * bb[0, t, h] * e[0, t, h] * np.outer(kt, kt @ Sm1)
                      - ratio * a[0, t - 1, h] * Sm2
                      + bb[0, t, h] * e[0, t, h] * np.outer(kt, v[0, t, h]))
                assert _rel(O[0, t, h], St.T @ q[0, t, h]) < 1e-10
                Sm2, Sm1 = Sm1, St
            assert _rel(ST[0, h], Sm1) < 1e-10


# --------------------------------------------------------------------------
# P8: DeltaNet's published chunk algorithm ([PDN slides] "Two keys still
# admit the compact delta-rule algorithm", Eq. (6), with the write key equal
# to the read key) at alpha = 1, mu = 0
# --------------------------------------------------------------------------
def _deltanet_chunk(q, k, v, beta, C, S_in):
    """S in R^{dv x dk}.  Per chunk:
    T = [I + tril(Diag(beta) K K^T, -1)]^{-1} Diag(beta), W = T K, U = T V,
    R = U - W S_in^T, S_out = S_in + R^T K, O = Q S_in^T + [(Q K^T) o Mask] R."""
    T_, Dk = k.shape
    O = np.zeros((T_, v.shape[1]))
    S = S_in.copy()
    for t0 in range(0, T_, C):
        sl = slice(t0, min(T_, t0 + C))
        K, Q, V, bt = k[sl], q[sl], v[sl], beta[sl]
        n = K.shape[0]
        Tm = np.linalg.inv(np.eye(n) + np.tril(np.diag(bt) @ K @ K.T, -1)) @ np.diag(bt)
        W, U = Tm @ K, Tm @ V
        R = U - W @ S.T
        O[sl] = Q @ S.T + ((Q @ K.T) * np.tril(np.ones((n, n)))) @ R
        S = S + R.T @ K
    return O, S


def pin_deltanet_chunk(lib):
    rng = np.random.default_rng(20)
    T, Dk, Dv = 37, 8, 6
    q = rng.standard_normal((1, T, 1, Dk))
    k = _unit_rows(rng, (1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    e = rng.uniform(0.05, 1.0, (1, T, 1))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    O, ST, _ = oracle.recurrence(q, k, v, np.ones_like(e), np.zeros_like(e), e, None, S0, None,
                                 lib=lib)
    for C in (4, 16):
        Od, Sd = _deltanet_chunk(q[0, :, 0], k[0, :, 0], v[0, :, 0], e[0, :, 0], C, S0[0, 0].T)
        assert _rel(O[0, :, 0], Od) < 1e-11
        assert _rel(ST[0, 0], Sd.T) < 1e-11


# --------------------------------------------------------------------------
# P9: structural invariants of the operator ([MDN slides] "Chunk outputs
# combine incoming states and local writes": two final states pass onward)
# --------------------------------------------------------------------------
def pin_gate_parameterisation(lib):
    """The coupled gates ([MDN slides] frame "Coupled gates restrict the
    spectral region"):
      - z_eta = 0 gives eta = 1, so alpha_max = 1 / (1 + s^2) and
        beta_max = s^2 / (1 + s^2) (cos^2 and sin^2 of arctan s);
      - z_alpha = -b gives softplus(0) = log 2, so alpha = alpha_max 2^-a;
        z_beta = 0 gives beta = beta_max / 2; z_mu = -b gives
        mu = max(2^-a, e^floor);
      - for any logits: 0 < eta < 2, alpha + beta <= 1, alpha <= alpha_max,
        mu <= 1 and log mu >= the floor;
      - z_mu -> -inf gives mu -> 1 and z_mu -> +inf gives mu = e^floor."""
    del lib
    tau, s, a, b, fl = 2.5, 1.7, 0.8, 0.3, -2.0
    kw = dict(tau=tau, s=s, a=a, b=b, log_mu_min=fl)
    al, mu, eta, be = oracle.gates_from_logits([0.0], [-b], [0.0], [-b], **kw)
    amax, bmax = 1.0 / (1.0 + s * s), s * s / (1.0 + s * s)
    assert abs(eta[0] - 1.0) < 1e-15
    assert _rel(al, [amax * 2.0 ** -a]) < 1e-14
    assert _rel(be, [bmax / 2.0]) < 1e-14
    assert _rel(mu, [max(2.0 ** -a, np.exp(fl))]) < 1e-14
    # off the centre: z_eta = tau artanh(1/2) gives eta = 3/2; z_alpha with
    # softplus(z_alpha + b) = 1 gives alpha = alpha_max e^-a; z_beta = log 3
    # gives sigmoid = 3/4
    al, mu, eta, be = oracle.gates_from_logits([tau * np.arctanh(0.5)], [np.log(np.e - 1) - b],
                                               [np.log(3.0)], [-b], **kw)
    x2 = (1.5 * s) ** 2
    assert _rel(eta, [1.5]) < 1e-14
    assert _rel(al, [np.exp(-a) / (1.0 + x2)]) < 1e-14
    assert _rel(be, [0.75 * x2 / (1.0 + x2)]) < 1e-14
    rng = np.random.default_rng(31)
    zs = [rng.normal(0.0, 4.0, 10000) for _ in range(4)]
    al, mu, eta, be = oracle.gates_from_logits(*zs, **kw)
    assert np.all(eta > 0.0) and np.all(eta < 2.0)
    assert np.all(al + be <= 1.0 + 1e-15)
    th = np.arctan(s * eta)
    assert np.all(al <= np.cos(th) ** 2 * (1 + 1e-15))
    assert np.all(mu <= 1.0) and np.all(np.log(mu) >= fl - 1e-12)
    _, mu_lo, _, _ = oracle.gates_from_logits([0.0], [0.0], [0.0], [-60.0], **kw)
    _, mu_hi, _, _ = oracle.gates_from_logits([0.0], [0.0], [0.0], [60.0], **kw)
    assert abs(mu_lo[0] - 1.0) < 1e-20 + a * np.exp(-60 + b) * 2
    assert _rel(mu_hi, [np.exp(fl)]) < 1e-15


def _fd_check(lib, inp, dO, dST, dMT, col_block, h=1e-6, tol=1e-8):
    """Central differences of L = <dO, O> + <dST, S_T> + <dMT, M_T> in every
    input element against recurrence_backward's gradient."""
    def loss(**over):
        x = dict(inp)
        x.update(over)
        O, ST, MT = oracle.recurrence(x["q"], x["k"], x["v"], x["alpha"], x["mu"], x["eta"],
                                      x["beta"], x["S0"], x["M0"], lib=lib)
        val = float(np.sum(O * dO))
        if dST is not None:
            val += float(np.sum(ST * dST))
        if dMT is not None:
            val += float(np.sum(MT * dMT))
        return val
    g = oracle.recurrence_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["mu"],
                                   inp["eta"], inp["beta"], inp["S0"], inp["M0"], dO=dO,
                                   dST=dST, dMT=dMT, col_block=col_block, lib=lib)
    for name, x in inp.items():
        if x is None:
            continue
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xp[idx] += h
            xm = x.copy()
            xm[idx] -= h
            fd[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
        got = g["d" + name]
        assert got is not None, name
        err = _rel(got, fd)
        assert err < tol, f"d{name}: finite differences disagree ({err:.2e})"


def pin_backward_finite_differences(lib):
    """The pages state the backward pass's strategy (save the residuals,
    rebuild the states) but no gradient formulas, so the reverse-mode
    derivative is pinned by its definition: central differences of a random
    linear functional of (O, S_T, M_T), element by element, for every input.
    Two cases: all four gates with initial states, terminal gradients and a
    ragged column block; beta = 1 (None), mu = 0, zero initial state and no
    terminal gradient."""
    rng = np.random.default_rng(41)
    B, T, H, Dk, Dv = 1, 5, 2, 3, 4
    a, m, e = _gates(rng, (B, T, H))
    inp = dict(q=rng.standard_normal((B, T, H, Dk)), k=rng.standard_normal((B, T, H, Dk)),
               v=rng.standard_normal((B, T, H, Dv)), alpha=a, mu=m, eta=e,
               beta=rng.uniform(0.2, 1.0, (B, T, H)), S0=rng.standard_normal((B, H, Dk, Dv)),
               M0=rng.standard_normal((B, H, Dk, Dv)))
    _fd_check(lib, inp, rng.standard_normal((B, T, H, Dv)),
              rng.standard_normal((B, H, Dk, Dv)), rng.standard_normal((B, H, Dk, Dv)),
              col_block=3)
    inp.update(beta=None, mu=np.zeros((B, T, H)), S0=None, M0=None)
    _fd_check(lib, inp, rng.standard_normal((B, T, H, Dv)), None, None, col_block=16)


def pin_layer_prologue_epilogue(lib):
    """The elementwise steps around the core ([MDN notes] Sec. 2.9):
      - prologue: q = (3, 4, 0, ..) normalises to (0.6, 0.8, 0, ..) as eps -> 0,
        and |x / sqrt(|x|^2 + eps)|^2 = |x|^2 / (|x|^2 + eps) exactly; the
        correction with d_h = 1 and q = k gives a zero query; d = 0 is no
        correction; the output keeps the direction of q - d_h k;
      - epilogue: o = (3, 4) has mean square 12.5, so g = 0 and w = (1, 2)
        give (0.5 * 3 / sqrt(12.5 + eps), 0.5 * 2 * 4 / sqrt(12.5 + eps));
        sigmoid(g) -> 1 for large g; RMSNorm is invariant to o -> c o (c > 0)
        as eps -> 0."""
    del lib
    q = np.zeros((1, 1, 8))
    q[0, 0, :2] = (3.0, 4.0)
    qo, ko = oracle.qk_prologue(q, q, None, eps=0.0)
    assert _rel(qo[0, 0, :2], [0.6, 0.8]) < 1e-15 and _rel(ko, qo) < 1e-15
    rng = np.random.default_rng(51)
    x = rng.standard_normal((5, 3, 16))
    kx = rng.standard_normal((5, 3, 16))
    eps = 0.37
    qo, ko = oracle.qk_prologue(x, kx, None, eps=eps)
    n2 = np.sum(x * x, axis=-1)
    assert _rel(np.sum(qo * qo, axis=-1), n2 / (n2 + eps)) < 1e-14
    d = np.array([1.0, 0.0, -0.5])
    qo, _ = oracle.qk_prologue(kx, kx, d, eps=1e-6)
    assert np.max(np.abs(qo[:, 0])) < 1e-12                     # d_h = 1, q = k
    qd, _ = oracle.qk_prologue(x, kx, d, eps=1e-9)
    want = x - d[:, None] * kx
    cos = np.sum(qd * want, -1) / (np.linalg.norm(qd, axis=-1) * np.linalg.norm(want, axis=-1))
    assert np.max(np.abs(cos - 1.0)) < 1e-12
    q0, _ = oracle.qk_prologue(x, kx, np.zeros(3), eps=eps)
    q1, _ = oracle.qk_prologue(x, kx, None, eps=eps)
    assert _rel(q0, q1) == 0.0
    y = oracle.output_epilogue([[3.0, 4.0]], [[0.0, 0.0]], [1.0, 2.0], eps=eps)
    r = np.sqrt(12.5 + eps)
    assert _rel(y, [[0.5 * 3.0 / r, 0.5 * 2.0 * 4.0 / r]]) < 1e-15
    o = rng.standard_normal((4, 2, 16))
    y1 = oracle.output_epilogue(o, np.full(o.shape, 40.0), None, eps=1e-12)
    y2 = oracle.output_epilogue(3.5 * o, np.full(o.shape, 40.0), None, eps=1e-12)
    assert _rel(y1, y2) < 1e-10
    assert _rel(np.mean(y1 * y1, axis=-1), np.ones((4, 2))) < 1e-10


def pin_invariants(lib):
    rng = np.random.default_rng(21)
    B, T, H, Dk, Dv = 2, 29, 2, 6, 7
    q, k, v, a, m, e, _, S0, M0 = _random_problem(rng, B, T, H, Dk, Dv)
    O, ST, MT = oracle.recurrence(q, k, v, a, m, e, None, S0, M0, lib=lib)
    # state passing: a split at T1 continued from (S_T1, M_T1) is the same run
    for T1 in (1, 11, 28):
        O1, S1, M1 = oracle.recurrence(q[:, :T1], k[:, :T1], v[:, :T1], a[:, :T1], m[:, :T1],
                                       e[:, :T1], None, S0, M0, lib=lib)
        O2, S2, M2 = oracle.recurrence(q[:, T1:], k[:, T1:], v[:, T1:], a[:, T1:], m[:, T1:],
                                       e[:, T1:], None, S1, M1, lib=lib)
        assert _rel(np.concatenate([O1, O2], axis=1), O) < TOL
        assert _rel(S2, ST) < TOL and _rel(M2, MT) < TOL
    # linearity in (V, S0, M0) jointly for fixed q, k and gates
    v2 = rng.standard_normal(v.shape)
    S2 = rng.standard_normal(S0.shape)
    M2 = rng.standard_normal(M0.shape)
    Ob, Sb, Mb = oracle.recurrence(q, k, v2, a, m, e, None, S2, M2, lib=lib)
    Oc, Sc, Mc = oracle.recurrence(q, k, 2.0 * v - 3.0 * v2, a, m, e, None, 2.0 * S0 - 3.0 * S2,
                                   2.0 * M0 - 3.0 * M2, lib=lib)
    assert _rel(Oc, 2.0 * O - 3.0 * Ob) < 1e-11
    assert _rel(Sc, 2.0 * ST - 3.0 * Sb) < 1e-11 and _rel(Mc, 2.0 * MT - 3.0 * Mb) < 1e-11
    # value columns are independent: a column subset is the same computation
    cols = [1, 4, 6]
    Os, Ss, Ms = oracle.recurrence(q, k, v[..., cols], a, m, e, None, S0[..., cols],
                                   M0[..., cols], lib=lib)
    assert _rel(Os, O[..., cols]) < TOL and _rel(Ss, ST[..., cols]) < TOL
    # heads and batch entries are independent
    Oh, Sh, Mh = oracle.recurrence(q[1:, :, 1:], k[1:, :, 1:], v[1:, :, 1:], a[1:, :, 1:],
                                   m[1:, :, 1:], e[1:, :, 1:], None, S0[1:, 1:], M0[1:, 1:],
                                   lib=lib)
    assert _rel(Oh, O[1:, :, 1:]) < TOL and _rel(Mh, MT[1:, 1:]) < TOL
    # the column-block split used for threading does not change the result
    Ob1, Sb1, Mb1 = oracle.recurrence(q, k, v, a, m, e, None, S0, M0, col_block=3, lib=lib)
    assert np.array_equal(Ob1, O) and np.array_equal(Sb1, ST) and np.array_equal(Mb1, MT)
    # decode steps chained equal the forward over the same tokens
    S, M = S0, M0
    for t in range(T):
        o, S, M = oracle.decode_step(q[:, t], k[:, t], v[:, t], a[:, t], m[:, t], e[:, t], S, M,
                                     lib=lib)
        assert _rel(o, O[:, t]) < TOL
    assert _rel(S, ST) < TOL and _rel(M, MT) < TOL


ALL_PINS = [pin_gate_parameterisation, pin_residuals, pin_layer_prologue_epilogue, pin_backward_finite_differences, 
    pin_one_token,
    pin_two_tokens,
    pin_gdn_reduction,
    pin_exact_recall,
    pin_chunk_equations,
    pin_gamma_forms_agree,
    pin_flagged_readings_fail,
    pin_frozen_step,
    pin_second_order,
    pin_deltanet_chunk,
    pin_invariants,
]
