"""Pins of the oracle's LQ-SGD step with K workers (CPU only).

Each worker compresses its own error-corrected gradient M_w = G_w + E_w from its own warm start
("Core claim" of the LQ-SGD review); the messages are log codes plus column maxima, which are
exchanged whole; the approximate global gradient (referee minor comment on Section III-A) is
the mean of the decoded messages, and error feedback ("What carries the argument") is taken
against it.  Checked here against the single-worker step (itself pinned in test_oracle_lq.py),
an independent decode of the codes from 60-digit decimal levels, numpy products, and the
bookkeeping identities of error feedback.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

getcontext().prec = 60
ALPHA = 10.0


def _levels(alpha, bits):
    """Decode levels ((1+alpha)^(k/L) - 1)/alpha to the nearest fp32, from decimal arithmetic."""
    L = (1 << (bits - 1)) - 1
    a = Decimal(alpha)
    out = []
    for k in range(L + 1):
        d = ((1 + a) ** (Decimal(k) / Decimal(L)) - 1) / a
        f = np.float32(float(d))
        best = f
        for c in (np.nextafter(f, np.float32(-1)), np.nextafter(f, np.float32(2))):
            if abs(Decimal(float(c)) - d) < abs(Decimal(float(best)) - d):
                best = c
        out.append(best)
    return np.array(out, np.float32)


def _decode(codes, colmax, alpha, bits):
    """sign(code) * fp32(level(|code|) * column maximum): one fp32 multiply per entry."""
    lv = _levels(alpha, bits)
    mag = lv[np.abs(codes.astype(np.int32))] * colmax[None, :].astype(np.float32)
    return np.where(codes < 0, -mag, mag).astype(np.float32)


def _workers(rng, K, n, m, r, spread=True):
    """K distinct workers; worker w's gradient is scaled by 4^w so that a wrong worker's message
    or a missing one is far outside rounding."""
    Gs, Es, Qs = [], [], []
    for w in range(K):
        s = 4.0 ** w if spread else 1.0
        Gs.append((rng.standard_normal((n, m)) * s).astype(np.float32))
        Es.append((rng.standard_normal((n, m)) * 0.1 * s).astype(np.float32))
        Qs.append(rng.standard_normal((m, r)).astype(np.float32))
    return Gs, Es, Qs


def _ulp_close(a, b, ulps=1):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    tol = ulps * np.spacing(np.maximum(np.abs(a), np.abs(b)))
    return np.all(np.abs(a.astype(np.float64) - b.astype(np.float64)) <= tol)


def test_one_worker_is_the_single_step(orc):
    rng = np.random.default_rng(70)
    n, m, r = 60, 44, 3
    Gs, Es, Qs = _workers(rng, 1, n, m, r)
    out = orc.lq_step_workers(Gs, Es, Qs, ALPHA, 8)
    one = orc.powersgd_logquant(Gs[0], Es[0], Qs[0], ALPHA, 8)
    assert np.array_equal(out["E"][0], one["E"]) and np.array_equal(out["Q"][0], one["Q"])
    for key in ("p_codes", "p_colmax", "q_codes", "q_colmax"):
        assert np.array_equal(out[key][0], one[key]), key
    ghat = one["p_hat"].astype(np.float64) @ one["Q"].astype(np.float64).T
    assert _ulp_close(out["G_hat"], ghat.astype(np.float32))


@pytest.mark.parametrize("bp,bq", [(8, 8), (8, 4)])
def test_each_worker_compresses_alone(orc, bp, bq):
    """Worker w's message and warm start are the single-worker step on (G_w, E_w, Q_w) alone."""
    rng = np.random.default_rng(71 + bq)
    K, n, m, r = 3, 50, 37, 4
    Gs, Es, Qs = _workers(rng, K, n, m, r)
    out = orc.lq_step_workers(Gs, Es, Qs, ALPHA, bp, bits_q=bq)
    for w in range(K):
        one = orc.powersgd_logquant(Gs[w], Es[w], Qs[w], ALPHA, bp, bits_q=bq)
        assert np.array_equal(out["Q"][w], one["Q"]), w
        for key in ("p_codes", "p_colmax", "q_codes", "q_colmax"):
            assert np.array_equal(out[key][w], one[key]), (w, key)


@pytest.mark.parametrize("K,bp,bq", [(2, 8, 8), (3, 8, 4), (5, 6, 8)])
def test_ghat_is_the_mean_of_the_decoded_messages(orc, K, bp, bq):
    """G_hat from the transmitted codes and maxima alone, decoded with levels from decimal
    arithmetic: fp32((1/K) sum_w Phat_w Qhat_w^T); the warm starts are the decoded Q factors."""
    rng = np.random.default_rng(80 + K)
    n, m, r = 45, 52, 3
    Gs, Es, Qs = _workers(rng, K, n, m, r)
    out = orc.lq_step_workers(Gs, Es, Qs, ALPHA, bp, bits_q=bq)
    total = np.zeros((n, m))
    for w in range(K):
        ph = _decode(out["p_codes"][w], out["p_colmax"][w], ALPHA, bp)
        qh = _decode(out["q_codes"][w], out["q_colmax"][w], ALPHA, bq)
        assert np.array_equal(qh, out["Q"][w]), w
        total += ph.astype(np.float64) @ qh.astype(np.float64).T
    assert _ulp_close(out["G_hat"], (total / K).astype(np.float32))
    # not the product of the mean factors (cross terms), nor the plain sum
    assert not _ulp_close(out["G_hat"], total.astype(np.float32), ulps=1000)


def test_error_feedback_uses_the_global_estimate(orc):
    """E_w <- M_w - G_hat for every worker (rounded once), so that
    sum_w E_w + K G_hat = sum_w M_w; the worker's own reconstruction is not what is subtracted."""
    rng = np.random.default_rng(90)
    K, n, m, r = 4, 40, 33, 2
    Gs, Es, Qs = _workers(rng, K, n, m, r)
    out = orc.lq_step_workers(Gs, Es, Qs, ALPHA, 8)
    total = np.zeros((n, m))
    for w in range(K):
        total += (_decode(out["p_codes"][w], out["p_colmax"][w], ALPHA, 8).astype(np.float64)
                  @ _decode(out["q_codes"][w], out["q_colmax"][w], ALPHA, 8).astype(np.float64).T)
    mean = total / K
    Ms = [(G + E).astype(np.float64) for G, E in zip(Gs, Es)]  # fp32 sums, exact in fp64
    for w in range(K):
        assert _ulp_close(out["E"][w], (Ms[w] - mean).astype(np.float32)), w
    lhs = sum(E.astype(np.float64) for E in out["E"]) + K * out["G_hat"].astype(np.float64)
    scale = max(np.abs(M).max() for M in Ms)
    assert np.abs(lhs - sum(Ms)).max() < 1e-6 * K * scale
    own = (_decode(out["p_codes"][0], out["p_colmax"][0], ALPHA, 8).astype(np.float64)
           @ _decode(out["q_codes"][0], out["q_colmax"][0], ALPHA, 8).astype(np.float64).T)
    assert np.abs(out["E"][0] - (Ms[0] - own)).max() > 1e-3 * np.abs(Ms[0]).max()


def test_identical_workers_reduce_to_one(orc):
    """K copies of one worker: every message is the single step's, G_hat its decoded product
    and every error its error, to fp32 rounding."""
    rng = np.random.default_rng(91)
    K, n, m, r = 4, 36, 28, 3
    G = rng.standard_normal((n, m)).astype(np.float32)
    E = (0.1 * rng.standard_normal((n, m))).astype(np.float32)
    Q = rng.standard_normal((m, r)).astype(np.float32)
    out = orc.lq_step_workers([G] * K, [E] * K, [Q] * K, ALPHA, 8)
    one = orc.powersgd_logquant(G, E, Q, ALPHA, 8)
    for w in range(K):
        for key in ("p_codes", "p_colmax", "q_codes", "q_colmax"):
            assert np.array_equal(out[key][w], one[key])
        assert np.array_equal(out["Q"][w], one["Q"])
        assert _ulp_close(out["E"][w], one["E"], ulps=2)
    ghat = one["p_hat"].astype(np.float64) @ one["Q"].astype(np.float64).T
    assert _ulp_close(out["G_hat"], ghat.astype(np.float32), ulps=2)


def test_error_feedback_telescopes_over_steps_and_workers(orc):
    """sum_t K G_hat_t + sum_w E_{w,T} = sum_t sum_w G_{w,t} + sum_w E_{w,0}: nothing is lost
    over steps and workers, only delayed."""
    rng = np.random.default_rng(92)
    K, n, m, r, T = 3, 32, 24, 2, 4
    Gs, Es, Qs = _workers(rng, K, n, m, r, spread=False)
    applied = np.zeros((n, m))
    fed = sum(E.astype(np.float64) for E in Es)
    for t in range(T):
        Gs = [rng.standard_normal((n, m)).astype(np.float32) for _ in range(K)]
        out = orc.lq_step_workers(Gs, Es, Qs, ALPHA, 8)
        applied += K * out["G_hat"].astype(np.float64)
        fed += sum(G.astype(np.float64) for G in Gs)
        Es, Qs = out["E"], out["Q"]
    resid = applied + sum(E.astype(np.float64) for E in Es) - fed
    assert np.abs(resid).max() < 1e-5 * np.abs(fed).max()


def test_message_size_per_worker(orc):
    """Each worker sends r(n b_p + m b_q) bits of codes and 2r fp32 maxima: with b = 8, a
    quarter of PowerSGD's fp32 factors."""
    rng = np.random.default_rng(93)
    K, n, m, r = 2, 30, 20, 4
    Gs, Es, Qs = _workers(rng, K, n, m, r)
    out = orc.lq_step_workers(Gs, Es, Qs, ALPHA, 8)
    assert out["p_codes"].shape == (K, n, r) and out["q_codes"].shape == (K, m, r)
    per_worker = (out["p_codes"].nbytes + out["q_codes"].nbytes) // K
    assert per_worker * 8 == r * (n + m) * 8
    assert per_worker / (4 * r * (n + m)) == 0.25
    assert out["p_colmax"].shape == (K, r) and out["q_colmax"].shape == (K, r)
