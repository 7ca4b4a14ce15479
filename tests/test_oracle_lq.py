"""Pins of the oracle's LQ-SGD step (CPU only).

Log quantiser (LQ-SGD review, "Core claim" Eq. 5 and referee major comment 1, Eq. 6): checked
against an independent 60-digit decimal evaluation of the bin boundaries and decode levels.
Power step: Gram-Schmidt against LAPACK's Householder QR, products against numpy, the exact
rank-1 case, error feedback (E_t = G'_t - Ghat_t) by its telescoping identity, and the payload
arithmetic r(n+m) b bits.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

getcontext().prec = 60


def _nearest_f32(d: Decimal) -> np.float32:
    f = np.float32(float(d))
    best = f
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        if abs(Decimal(float(c)) - d) < abs(Decimal(float(best)) - d):
            best = c
    return best


def _f32_below_above(d: Decimal):
    f = np.float32(float(d))
    while Decimal(float(f)) >= d:
        f = np.nextafter(f, np.float32(-np.inf))
    lo = f
    hi = np.nextafter(lo, np.float32(np.inf))
    assert Decimal(float(hi)) >= d
    return lo, hi


def _boundary(k, alpha, L):
    a = Decimal(alpha)
    z = (Decimal(2 * k + 1) / Decimal(2 * L))
    return ((1 + a) ** z - 1) / a


def _level(k, alpha, L):
    a = Decimal(alpha)
    return ((1 + a) ** (Decimal(k) / Decimal(L)) - 1) / a


@pytest.mark.parametrize("alpha,bits", [(10.0, 8), (1.0, 8), (100.0, 8), (10.0, 4)])
def test_log_bins_match_high_precision_boundaries(orc, alpha, bits):
    L = 2 ** (bits - 1) - 1
    for k in range(L):
        b = _boundary(k, alpha, L)
        lo, hi = _f32_below_above(b)
        # no fp32 lies on (or within 1e-12 of) a boundary, so ties never arise
        assert (b - Decimal(float(lo))) / b > Decimal("1e-12")
        assert (Decimal(float(hi)) - b) / b > Decimal("1e-12")
        assert orc.logq_index(lo, alpha, L) == k
        assert orc.logq_index(hi, alpha, L) == k + 1


@pytest.mark.parametrize("alpha,bits", [(10.0, 8), (1.0, 8), (10.0, 4)])
def test_log_levels_match_high_precision(orc, alpha, bits):
    L = 2 ** (bits - 1) - 1
    for k in range(L + 1):
        assert orc.logq_level(k, alpha, L) == _nearest_f32(_level(k, alpha, L))
    assert orc.logq_level(0, alpha, L) == 0.0
    assert orc.logq_level(L, alpha, L) == 1.0


def test_log_quantiser_closed_forms(orc):
    alpha, L = 10.0, 127
    assert orc.logq_index(0.0, alpha, L) == 0
    assert orc.logq_index(1.0, alpha, L) == L
    ys = np.sort(np.random.default_rng(0).uniform(0, 1, 20000).astype(np.float32))
    idx = [orc.logq_index(float(y), alpha, L) for y in ys]
    assert all(a <= b for a, b in zip(idx, idx[1:]))
    # every decode level encodes back to itself
    for k in range(L + 1):
        assert orc.logq_index(orc.logq_level(k, alpha, L), alpha, L) == k


def test_logquant_normalises_large_entries(orc):
    rng = np.random.default_rng(1)
    F = (rng.standard_normal((300, 3)) * np.array([1e6, 1.0, 1e-6])).astype(np.float32)
    F[:, 2] *= 0  # a zero column
    codes, colmax, Fhat = orc.logquant(F, 10.0, 8)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    assert np.array_equal(colmax, np.abs(F).max(0))
    for c in range(2):
        i = np.abs(F[:, c]).argmax()
        assert abs(int(codes[i, c])) == 127
        assert Fhat[i, c] == F[i, c]
    assert not codes[:, 2].any() and not Fhat[:, 2].any()
    assert np.array_equal(np.sign(codes[:, :2]), np.sign(F[:, :2]).astype(np.int8) *
                          (codes[:, :2] != 0))


def test_mgs_matches_householder_qr(orc):
    rng = np.random.default_rng(2)
    for n, r in ((64, 1), (500, 4), (1000, 7)):
        P = rng.standard_normal((n, r)).astype(np.float32)
        got = orc.mgs(P, 1000)
        q, R = np.linalg.qr(P.astype(np.float64))
        q = q * np.sign(np.diag(R))
        assert np.abs(got - q).max() < 1e-6
        assert np.abs(got.T.astype(np.float64) @ got - np.eye(r)).max() < 1e-6


def test_mgs_zero_column_stays_zero(orc):
    rng = np.random.default_rng(3)
    P = rng.standard_normal((50, 3)).astype(np.float32)
    P[:, 1] = 0
    got = orc.mgs(P, 1000)
    assert not got[:, 1].any()
    assert abs(np.linalg.norm(got[:, 2].astype(np.float64)) - 1) < 1e-6


def test_mgs_dependent_columns_are_zero(orc):
    """A column that is a combination of earlier ones up to fp32 rounding has nothing of its
    own left after the projections; it is set to zero like an exactly zero column, and the
    columns after it are still orthonormalised against the live ones.  A column with a small
    but real component of its own (1e-3 of its norm) stays."""
    rng = np.random.default_rng(31)
    n = 400
    P = rng.standard_normal((n, 6)).astype(np.float32)
    P[:, 1] = 3.0 * P[:, 0]                        # exactly dependent
    P[:, 3] = (P[:, 0] + P[:, 2]).astype(np.float32)  # dependent up to fp32 rounding
    W = rng.standard_normal(n)
    P[:, 4] = (P[:, 2] + 1e-3 * W).astype(np.float32)  # a small part of its own
    got = orc.mgs(P, 1000).astype(np.float64)
    assert not got[:, 1].any() and not got[:, 3].any()
    live = [0, 2, 4, 5]
    assert np.abs(got[:, live].T @ got[:, live] - np.eye(4)).max() < 1e-6
    # the live columns span what the original ones span
    q, _ = np.linalg.qr(P[:, live].astype(np.float64))
    assert np.abs(got[:, live] - q @ (q.T @ got[:, live])).max() < 1e-6


def _bound_and_rest(P):
    """For the last column of an fp32 P (taken exactly in fp64): the norm it keeps after
    projecting out the earlier columns, and |p_c| + sum_j |a_j| |p_j| with a its coefficients
    on the earlier columns."""
    P64 = P.astype(np.float64)
    A, c = P64[:, :-1], P64[:, -1]
    a, *_ = np.linalg.lstsq(A, c, rcond=None)
    rest = np.linalg.norm(c - A @ a)
    bound = np.linalg.norm(c) + np.sum(np.abs(a) * np.linalg.norm(A, axis=0))
    return rest, bound


def _column_at(rng, n, coef, frac, rho, ill=False):
    """fp32 columns p_0, p_1 and p_2 = coef_0 p_0 + coef_1 p_1 + t w, w orthogonal to p_0 and
    p_1, with t = frac * rho * (|p_2| + |coef_0| |p_0| + |coef_1| |p_1|).  ill: p_1 = p_0 plus
    1/100 of a direction of its own (nearly parallel earlier columns)."""
    A = rng.standard_normal((n, 2))
    if ill:
        A[:, 1] = A[:, 0] + 0.01 * rng.standard_normal(n)
    A = A.astype(np.float32).astype(np.float64)
    w = rng.standard_normal(n)
    qa, _ = np.linalg.qr(A)
    w -= qa @ (qa.T @ w)
    w /= np.linalg.norm(w)
    base = A @ np.asarray(coef, np.float64)
    bound = np.linalg.norm(base) + np.sum(np.abs(coef) * np.linalg.norm(A, axis=0))
    P = np.empty((n, 3), np.float32)
    P[:, :2] = A
    P[:, 2] = base + frac * rho * bound * w
    rest, bound = _bound_and_rest(P)
    return P, rest / (rho * bound)


@pytest.mark.parametrize("m", [1024, 11008])
@pytest.mark.parametrize("ill", [False, True])
def test_mgs_cut_from_fp32_rounding(orc, m, ill):
    """The dependent-column cut follows from fp32 arithmetic alone: a column whose remaining
    norm is at most rho (|p_c| + sum_j |a_j| |p_j|), rho = sqrt(m) 2^-24, is set to zero and one
    with a little more is kept -- with well-separated earlier columns (coefficients (1, 0.5))
    and with nearly parallel ones (coefficients (-49, 50), where the bound is ~90 times the
    column's own norm: a cut without the coefficient term would keep the column that must
    go)."""
    rho = np.sqrt(m) * 2.0 ** -24
    assert orc.mgs_rho(m) == rho
    rng = np.random.default_rng(m + ill)
    coef = (-49.0, 50.0) if ill else (1.0, 0.5)
    for frac, kept in ((1.15, True), (0.87, False), (2.0, True), (0.5, False)):
        P, ratio = _column_at(rng, 400, coef, frac, rho, ill)
        assert abs(ratio / frac - 1.0) < 0.04, (ratio, frac)
        got = orc.mgs(P, m).astype(np.float64)
        if kept:
            assert abs(np.linalg.norm(got[:, 2]) - 1.0) < 1e-6
            assert np.abs(got.T @ got - np.eye(3)).max() < 1e-6
        else:
            assert not got[:, 2].any()
            assert np.abs(got[:, :2].T @ got[:, :2] - np.eye(2)).max() < 1e-6


def _step(orc, G, E, Q):
    return orc.powersgd_logquant(G, E, Q, 10.0, 8)


def test_power_step_against_numpy(orc):
    rng = np.random.default_rng(4)
    n, m, r = 96, 80, 3
    G = rng.standard_normal((n, m)).astype(np.float32)
    E = (rng.standard_normal((n, m)) * 0.1).astype(np.float32)
    Q = rng.standard_normal((m, r)).astype(np.float32)
    out = _step(orc, G, E, Q)
    Mf = (G + E).astype(np.float64)  # G + E rounded in fp32 is what the step works on
    Ghat = out["p_hat"].astype(np.float64) @ out["Q"].T.astype(np.float64)
    assert np.abs(out["E"] + Ghat - Mf).max() < 1e-6 * np.abs(Mf).max()
    q, R = np.linalg.qr(Mf @ Q.astype(np.float64))
    q = q * np.sign(np.diag(R))
    assert np.abs(out["P_pre"] - q).max() < 1e-5
    Qref = Mf.T @ out["P_pre"].astype(np.float64)
    assert np.abs(out["Q_pre"] - Qref).max() <= 1e-6 * np.abs(Qref).max()
    # Q leaves the step as the decoded factor, identical to quantising Q_pre
    codes, cmax, Qhat = orc.logquant(out["Q_pre"], 10.0, 8)
    assert np.array_equal(out["Q"], Qhat)
    assert np.array_equal(out["q_codes"], codes) and np.array_equal(out["q_colmax"], cmax)
    codes, cmax, Phat = orc.logquant(out["P_pre"], 10.0, 8)
    assert np.array_equal(out["p_hat"], Phat) and np.array_equal(out["p_codes"], codes)


def test_power_step_exact_rank_one(orc):
    rng = np.random.default_rng(5)
    n, m = 200, 150
    u = rng.standard_normal(n)
    v = rng.standard_normal(m)
    G = np.outer(u, v).astype(np.float32)
    E = np.zeros_like(G)
    Q = rng.standard_normal((m, 1)).astype(np.float32)
    out = _step(orc, G, E, Q)
    M = G.astype(np.float64)
    before = out["P_pre"].astype(np.float64) @ out["Q_pre"].astype(np.float64).T
    assert np.abs(before - M).max() < 1e-5 * np.abs(M).max()
    after = out["p_hat"].astype(np.float64) @ out["Q"].astype(np.float64).T
    rel = np.linalg.norm(after - M) / np.linalg.norm(M)
    assert rel < 0.03
    # M = Ghat + E to fp32 rounding
    assert np.abs(after + out["E"] - M).max() < 1e-6 * np.abs(M).max()


def test_error_feedback_telescopes(orc):
    """sum_t Ghat_t + E_T = sum_t G_t + E_0 (nothing is lost, only delayed)."""
    rng = np.random.default_rng(6)
    n, m, r, T = 64, 48, 2, 3
    E = np.zeros((n, m), np.float32)
    Q = rng.standard_normal((m, r)).astype(np.float32)
    sum_hat = np.zeros((n, m))
    sum_g = np.zeros((n, m))
    for t in range(T):
        G = rng.standard_normal((n, m)).astype(np.float32)
        out = _step(orc, G, E, Q)
        sum_hat += out["p_hat"].astype(np.float64) @ out["Q"].astype(np.float64).T
        sum_g += G
        E, Q = out["E"], out["Q"]
    assert np.abs(sum_hat + E - sum_g).max() < 1e-5 * np.abs(sum_g).max()
    # the error is smaller than the signal (the compressor is a contraction here)
    assert np.linalg.norm(E) < np.linalg.norm(sum_g)


def test_payload_bits(orc):
    """r(n+m) b-bit indices, 32/b smaller than fp32 factors (a 75% cut at b = 8)."""
    rng = np.random.default_rng(7)
    n, m, r = 40, 30, 4
    out = _step(orc, rng.standard_normal((n, m)).astype(np.float32), np.zeros((n, m), np.float32),
                rng.standard_normal((m, r)).astype(np.float32))
    code_bytes = out["p_codes"].nbytes + out["q_codes"].nbytes
    assert code_bytes * 8 == r * (n + m) * 8
    assert 1 - code_bytes / (4 * r * (n + m)) == 0.75
    assert out["p_colmax"].nbytes + out["q_colmax"].nbytes == 8 * r


@pytest.mark.parametrize("bp,bq", [(8, 4), (4, 8), (3, 6)])
def test_separate_code_widths(orc, bp, bq):
    """b_p and b_q act on their own factors: the step's codes are exactly the log quantiser's
    codes of its unquantised P (width b_p) and Q (width b_q), each within its own range, and
    the error-feedback identity holds whatever the widths; the payload is r(n b_p + m b_q)
    bits."""
    rng = np.random.default_rng(40 + bp + bq)
    n, m, r = 50, 36, 3
    G = rng.standard_normal((n, m)).astype(np.float32)
    E = (0.1 * rng.standard_normal((n, m))).astype(np.float32)
    Q = rng.standard_normal((m, r)).astype(np.float32)
    out = orc.powersgd_logquant(G, E, Q, 10.0, bp, bits_q=bq)
    pc, pm, ph = orc.logquant(out["P_pre"], 10.0, bp)
    qc, qm, qh = orc.logquant(out["Q_pre"], 10.0, bq)
    assert np.array_equal(out["p_codes"], pc) and np.array_equal(out["q_codes"], qc)
    assert np.array_equal(out["p_hat"], ph) and np.array_equal(out["Q"], qh)
    assert np.abs(out["p_codes"]).max() == (1 << (bp - 1)) - 1
    assert np.abs(out["q_codes"]).max() == (1 << (bq - 1)) - 1
    M = G.astype(np.float64) + E
    ghat = out["p_hat"].astype(np.float64) @ out["Q"].astype(np.float64).T
    assert np.abs(ghat + out["E"] - M).max() < 1e-6 * np.abs(M).max()
    assert r * (n * bp + m * bq) == sum(int(np.ceil(np.log2(2 * ((1 << (b - 1)) - 1) + 1))) * c
                                        for b, c in ((bp, r * n), (bq, r * m)))


@pytest.mark.parametrize("r", [1, 4])
def test_error_feedback_stays_bounded_and_recovers(orc, r):
    """The review's falsifier for error feedback: the error matrix must not keep growing.  On a
    fixed gradient G, E_t rises while the compressor catches up and then stays flat, and the
    running mean of the decoded gradients converges to G like 1/T (sum_t Ghat_t = T G - E_T)."""
    rng = np.random.default_rng(50 + r)
    n, m = 64, 48
    G = rng.standard_normal((n, m)).astype(np.float32)
    E = np.zeros((n, m), np.float32)
    Q = rng.standard_normal((m, r)).astype(np.float32)
    total = np.zeros((n, m))
    err, mean_err = {}, {}
    for t in range(1, 201):
        out = orc.powersgd_logquant(G, E, Q, 10.0, 8)
        total += out["p_hat"].astype(np.float64) @ out["Q"].astype(np.float64).T
        E, Q = out["E"], out["Q"]
        if t in (100, 150, 200):
            err[t] = np.linalg.norm(E)
            mean_err[t] = np.linalg.norm(total / t - G)
    assert err[200] <= 1.1 * err[100] and err[150] <= 1.1 * err[100]
    assert mean_err[200] <= 0.6 * mean_err[100]
    assert mean_err[200] < 0.2 * np.linalg.norm(G)
