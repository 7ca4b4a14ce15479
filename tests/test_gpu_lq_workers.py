"""GPU parity of the LQ-SGD step with K workers (gq_lq_step_workers) against the CPU oracle.

Every worker's message (codes and column maxima of its P and Q'), its decoded warm start, its
new error and the common G_hat are compared within the single-worker step's tolerances: the
products and the orthonormalisation sum in a different order, so a factor value within
rounding of a bin boundary may code one bin apart (codes at most 1 apart, < 0.1% of them), and
the decoded matrices agree to a relative Frobenius error of 2e-3.  Each step starts both sides
from the oracle's state.  K = 1 must reproduce the single-worker entry point bit for bit.
"""
import numpy as np
import pytest
import torch

from allreduce_compatible_gradient_amd import workloads as W
from tests.gpu_helpers import dev, gq, host, say

pytestmark = pytest.mark.gpu
ALPHA, BITS = W.LQ_ALPHA, W.LQ_BITS


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _step_both(orc, Gs, Es, Qs, bp=BITS, bq=BITS):
    g = gq()
    ref = orc.lq_step_workers(Gs, Es, Qs, ALPHA, bp, bits_q=bq)
    Ed = [dev(E) for E in Es]
    Qd = [dev(Q) for Q in Qs]
    out = g.lq_step_workers([dev(G) for G in Gs], Ed, Qd, ALPHA, bp, bits_q=bq, want_pre=True)
    out["bits"] = (bp, bq)
    return ref, out, [host(E) for E in Ed], [host(Q) for Q in Qd]


def _check_requant(out, Qg):
    """Each worker's codes, column maxima and decoded warm start are what the oracle's
    quantiser gives on that worker's own unquantised factors from the GPU, bit for bit."""
    from oracle import oracle as orc
    bp, bq = out["bits"]
    alpha = out.get("alpha", ALPHA)
    P_pre, Q_pre = host(out["p_pre"]), host(out["q_pre"])
    pc, pm = host(out["p_codes"]), host(out["p_colmax"])
    qc, qm = host(out["q_codes"]), host(out["q_colmax"])
    for w in range(len(Qg)):
        rc, rm, _ = orc.logquant(P_pre[w], alpha, bp)
        assert np.array_equal(pc[w], rc), ("p_codes", w)
        assert np.array_equal(pm[w], rm), ("p_colmax", w)
        rc, rm, rh = orc.logquant(Q_pre[w], alpha, bq)
        assert np.array_equal(qc[w], rc), ("q_codes", w)
        assert np.array_equal(qm[w], rm), ("q_colmax", w)
        assert np.array_equal(Qg[w], rh), ("warm start", w)


def _check(ref, out, Eg, Qg, tol=2e-3):
    K = len(Eg)
    if "p_pre" in out:
        _check_requant(out, Qg)
    for key in ("p_codes", "q_codes"):
        gc = host(out[key]).astype(np.int32)
        rc = ref[key].astype(np.int32)
        assert gc.shape == rc.shape
        assert np.abs(gc - rc).max() <= 1, key
        assert np.mean(gc != rc) < 1e-3, key
    for key in ("p_colmax", "q_colmax"):
        np.testing.assert_allclose(host(out[key]), ref[key], rtol=1e-5)
    for w in range(K):
        assert _rel(Qg[w], ref["Q"][w]) < tol, ("Q", w)
        assert _rel(Eg[w], ref["E"][w]) < tol, ("E", w)
    assert _rel(host(out["G_hat"]), ref["G_hat"]) < tol


def _workers(rng, K, n, m, r):
    """Distinct workers: a shared rank-1 signal plus each worker's noise at its own scale."""
    u, v = rng.standard_normal(n), rng.standard_normal(m)
    Gs = [(np.outer(u, v) * 1e-3 + rng.standard_normal((n, m)) * 1e-3 * 2.0 ** (w % 3))
          .astype(np.float32) for w in range(K)]
    return Gs


@pytest.mark.parametrize("K,n,m,r,bp,bq", [(2, 300, 200, 1, 8, 8), (3, 257, 301, 7, 8, 8),
                                           (4, 64, 40, 8, 8, 4), (8, 1000, 999, 3, 8, 8),
                                           (5, 513, 260, 4, 6, 8), (16, 128, 96, 2, 8, 8)])
def test_workers_small(orc, K, n, m, r, bp, bq):
    say("lq workers small", K, n, m, r, bp, bq)
    rng = np.random.default_rng(K * 1000 + n + m + r)
    Es = [np.zeros((n, m), np.float32) for _ in range(K)]
    Qs = [rng.standard_normal((m, r)).astype(np.float32) for _ in range(K)]
    for t in range(3):
        Gs = _workers(rng, K, n, m, r)
        ref, out, Eg, Qg = _step_both(orc, Gs, Es, Qs, bp, bq)
        _check(ref, out, Eg, Qg)
        Es, Qs = ref["E"], ref["Q"]


def test_one_worker_is_the_single_step():
    """K = 1 through gq_lq_step_workers equals gq_powersgd_logquant bit for bit; its G_hat is
    the decoded product P_hat Q_hat^T."""
    g = gq()
    n, m, r = 700, 612, 5
    say("lq workers K=1 vs single step", n, m, r)
    gen = torch.Generator(device="cuda").manual_seed(21)
    G = torch.randn(n, m, device="cuda", generator=gen)
    E0 = torch.randn(n, m, device="cuda", generator=gen) * 0.1
    Q0 = torch.randn(m, r, device="cuda", generator=gen)
    E1, Q1 = E0.clone(), Q0.clone()
    one = g.powersgd_logquant(G, E1, Q1, ALPHA, BITS)
    E2, Q2 = E0.clone(), Q0.clone()
    out = g.lq_step_workers([G], [E2], [Q2], ALPHA, BITS)
    torch.cuda.synchronize()
    assert torch.equal(E1, E2) and torch.equal(Q1, Q2)
    for key in ("p_codes", "p_colmax", "q_codes", "q_colmax"):
        assert torch.equal(out[key][0], one[key]), key
    ghat = one["p_hat"].double() @ Q1.double().T
    assert (out["G_hat"].double() - ghat).abs().max().item() <= 1e-6 * ghat.abs().max().item()


def test_error_feedback_identity_on_gpu():
    """sum_w E_w(new) + K G_hat = sum_w (G_w + E_w(old)) to fp32 rounding, and each worker's
    warm start leaves as the log quantiser's decode of its own Q codes."""
    g = gq()
    K, n, m, r = 6, 512, 384, 4
    say("lq workers identity", K, n, m, r)
    gen = torch.Generator(device="cuda").manual_seed(22)
    Gs = [torch.randn(n, m, device="cuda", generator=gen) for _ in range(K)]
    Es = [torch.randn(n, m, device="cuda", generator=gen) * 0.1 for _ in range(K)]
    Qs = [torch.randn(m, r, device="cuda", generator=gen) for _ in range(K)]
    Msum = sum((G + E).double() for G, E in zip(Gs, Es))
    out = g.lq_step_workers(Gs, Es, Qs, ALPHA, BITS)
    lhs = sum(E.double() for E in Es) + K * out["G_hat"].double()
    assert (lhs - Msum).abs().max().item() < 1e-6 * K * Msum.abs().max().item()
    lv = torch.tensor([((1 + ALPHA) ** (k / 127) - 1) / ALPHA for k in range(128)],
                      dtype=torch.float64, device="cuda").float()
    for w in range(K):
        c = out["q_codes"][w].long()
        mag = lv[c.abs()] * out["q_colmax"][w][None, :]
        dec = torch.where(c < 0, -mag, mag)
        # levels from libm's pow in double rounded to fp32 agree with the table to 1 ulp
        assert torch.allclose(dec, Qs[w], rtol=2.5e-7, atol=0)


@pytest.mark.parametrize("K,shape,r", [(4, (4096, 4096), 7), (8, (4096, 11008), 1),
                                       (8, (4096, 4096), 1), (8, (4096, 4096), 7),
                                       (8, (4096, 11008), 7)])
def test_workers_full_shapes(orc, K, shape, r):
    """The LQ-SGD workload shapes with K workers (shared rank-8 signal, each worker's own noise),
    one step from zero error and the common Q_0; the last three are the benchmark's
    configurations, run through the same launches it times."""
    n, m = shape
    say("lq workers full", K, n, m, r)
    Gs, Qs = [], []
    for w in range(K):
        G, Q0 = W.lq_worker_problem(n, m, r, 0, w, "cpu")
        Gs.append(G.numpy())
        Qs.append(Q0.numpy())
    Es = [np.zeros((n, m), np.float32) for _ in range(K)]
    ref, out, Eg, Qg = _step_both(orc, Gs, Es, Qs)
    _check(ref, out, Eg, Qg)


@pytest.mark.parametrize("case", ["K=0", "K=17", "shared E", "shared Q", "G_hat is E", "r=9",
                                  "n too large"])
def test_argument_errors(case):
    """Refused on the host with GQ_EINVAL before anything is launched."""
    g = gq()
    say("lq workers error", case)
    if case == "K=0":
        ctx = g.context()
        rc = g._lib.gq_lq_step_workers(ctx.handle, None, None, None, 0, 32, 16, 2, ALPHA, BITS,
                                       BITS, None, None, None, None, None, None, None, None)
        assert rc == 1
        return
    n, m, r, K = 32, 16, 2, 3
    if case == "n too large":
        n, m, K = 65535 * 64 + 1, 1, 1
    Gs = [torch.zeros(n, m, device="cuda") for _ in range(K)]
    Es = [torch.zeros(n, m, device="cuda") for _ in range(K)]
    Qs = [torch.zeros(m, r, device="cuda") for _ in range(K)]
    out = {}
    if case == "K=17":
        Gs = [Gs[0]] * 17
        Es = [torch.zeros(n, m, device="cuda") for _ in range(17)]
        Qs = [torch.zeros(m, r, device="cuda") for _ in range(17)]
    elif case == "shared E":
        Es[2] = Es[0]
    elif case == "shared Q":
        Qs[1] = Qs[0]
    elif case == "G_hat is E":
        out["G_hat"] = Es[1]
    elif case == "r=9":
        Qs = [torch.zeros(m, 9, device="cuda") for _ in range(K)]
    with pytest.raises(g.GQError) as ei:
        g.lq_step_workers(Gs, Es, Qs, ALPHA, BITS, out=out)
    assert ei.value.code == 1  # GQ_EINVAL


@pytest.mark.parametrize("i", range(10))
def test_workers_random_configurations(orc, i):
    """Seeded random worker counts (1-16), shapes (m not always a multiple of 4), ranks 1-8,
    alpha in {1, 10, 100} and code widths b_p, b_q in 4..8; workers share a low-rank signal
    at their own scales; two steps each, within the step tolerances."""
    g = gq()
    rng = np.random.default_rng(80000 + i)
    K = int(rng.integers(1, 17))
    r = int(rng.integers(1, 9))
    n = int(rng.integers(max(r, 8), 1200))
    m = int(rng.integers(max(r, 8), 1200))
    alpha = float(rng.choice([1.0, 10.0, 100.0]))
    bp, bq = int(rng.integers(4, 9)), int(rng.integers(4, 9))
    say("lq workers random", i, K, n, m, r, alpha, bp, bq)
    U_ = rng.standard_normal((n, 8)) * 1e-3
    V_ = rng.standard_normal((m, 8))
    scale = 10.0 ** rng.uniform(-1, 1, K)
    Es = [np.zeros((n, m), np.float32) for _ in range(K)]
    Qs = [rng.standard_normal((m, r)).astype(np.float32) for _ in range(K)]
    for t in range(2):
        Gs = [((rng.standard_normal((n, m)) * 1e-3 + U_ @ V_.T) * scale[w]).astype(np.float32)
              for w in range(K)]
        ref = orc.lq_step_workers(Gs, Es, Qs, alpha, bp, bits_q=bq)
        Ed = [dev(E) for E in Es]
        Qd = [dev(Q) for Q in Qs]
        out = g.lq_step_workers([dev(G) for G in Gs], Ed, Qd, alpha, bp, bits_q=bq,
                                want_pre=True)
        out["bits"], out["alpha"] = (bp, bq), alpha
        _check(ref, out, [host(E) for E in Ed], [host(Q) for Q in Qd])
        Es, Qs = ref["E"], ref["Q"]
