"""The hot path under HIP graph capture.

After one eager call has sized a context's scratch and cached its tables, a call only
launches kernels, so the global norm + fused pass and the LQ-SGD step can be captured into a
graph and replayed.  Each test captures on a context of its own (a graph keeps pointers to
that context's scratch), replays several times with eager work and synchronisations in
between, and checks every replay against the same calls made eagerly: bit for bit, since the
kernels are deterministic.
"""
import numpy as np
import pytest
import torch

from allreduce_compatible_gradient_amd import workloads as W
from tests.gpu_helpers import dev, first_diff, gq, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def test_norm_and_fused_pass_in_a_graph(orc):
    g = gq()
    say("graph: norm + fused")
    w = W.reduced("resnet50-161t-f32-K8-exp7")
    xs = [x.to("cuda") for x in W.gradients(w, "cpu")]
    gctx, ectx = g.Context(), g.Context()
    S = torch.empty(w.nseg, dtype=torch.float32, device="cuda")
    out = torch.empty(w.n, dtype=torch.float32, device="cuda")

    def step(ctx, S_, out_):
        g.global_norm(xs, w.offsets, scale_out=S_, ctx=ctx)
        g.fused_mean(xs, S_, w.grid, w.levels, w.bits, 11, w.acc_bits, 0, offsets=w.offsets,
                     out=out_, ctx=ctx)

    step(gctx, S, out)                       # sizes the scratch, caches the segment table
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gctx, S, out)
    S_e = torch.empty_like(S)
    out_e = torch.empty_like(out)
    for rep in range(3):
        for x in xs:                         # eager work between replays: new gradients
            x.mul_(1.5 if rep % 2 == 0 else -0.75)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(ectx, S_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(S, S_e), "replay %d: scale" % rep
        assert torch.equal(out, out_e), "replay %d: %s" % (rep, first_diff(host(out), host(out_e)))
    # and the last replay against the oracle
    ref = orc.allreduce_mean([host(x) for x in xs], w.grid, w.levels, w.bits, w.acc_bits, 11, 0,
                             w.offsets, scale=host(S))
    assert np.array_equal(host(out), ref["mean"]), first_diff(host(out), ref["mean"])
    del graph
    gctx.close()
    ectx.close()


def test_lq_step_in_a_graph():
    g = gq()
    n, m, r = 1024, 768, 4
    say("graph: lq step", n, m, r)
    gen = torch.Generator(device="cuda").manual_seed(17)
    G = torch.randn(n, m, device="cuda", generator=gen) * 1e-3
    E0 = torch.randn(n, m, device="cuda", generator=gen) * 1e-4
    Q0 = torch.randn(m, r, device="cuda", generator=gen)
    gctx, ectx = g.Context(), g.Context()
    Eg, Qg = E0.clone(), Q0.clone()
    Ee, Qe = E0.clone(), Q0.clone()
    og = g.powersgd_logquant(G, Eg, Qg, W.LQ_ALPHA, W.LQ_BITS, ctx=gctx)   # warm-up: one step
    oe = g.powersgd_logquant(G, Ee, Qe, W.LQ_ALPHA, W.LQ_BITS, ctx=ectx)
    torch.cuda.synchronize()
    assert torch.equal(Eg, Ee) and torch.equal(Qg, Qe)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        og = g.powersgd_logquant(G, Eg, Qg, W.LQ_ALPHA, W.LQ_BITS, out=og, ctx=gctx)
    # capture does not run the step: both copies are still one step in
    torch.cuda.synchronize()
    for rep in range(4):
        G.mul_(-1.25)                          # a new gradient every step, eagerly
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe = g.powersgd_logquant(G, Ee, Qe, W.LQ_ALPHA, W.LQ_BITS, out=oe, ctx=ectx)
        torch.cuda.synchronize()
        for k in ("p_codes", "q_codes", "p_colmax", "q_colmax", "p_hat"):
            assert torch.equal(og[k], oe[k]), "replay %d: %s" % (rep, k)
        assert torch.equal(Eg, Ee), "replay %d: E" % rep
        assert torch.equal(Qg, Qe), "replay %d: Q" % rep
    del graph
    gctx.close()
    ectx.close()


def test_lq_workers_step_in_a_graph():
    """The K-worker LQ-SGD step captured after a warm-up call and replayed on fresh gradients:
    every replay equals the eager step on a second context bit for bit."""
    g = gq()
    K, n, m, r = 3, 640, 512, 3
    say("graph: lq workers step", K, n, m, r)
    gen = torch.Generator(device="cuda").manual_seed(18)
    Gs = [torch.randn(n, m, device="cuda", generator=gen) * 1e-3 for _ in range(K)]
    E0 = [torch.randn(n, m, device="cuda", generator=gen) * 1e-4 for _ in range(K)]
    Q0 = [torch.randn(m, r, device="cuda", generator=gen) for _ in range(K)]
    gctx, ectx = g.Context(), g.Context()
    Eg, Qg = [e.clone() for e in E0], [q.clone() for q in Q0]
    Ee, Qe = [e.clone() for e in E0], [q.clone() for q in Q0]
    og = g.lq_step_workers(Gs, Eg, Qg, W.LQ_ALPHA, W.LQ_BITS, ctx=gctx)   # warm-up: one step
    oe = g.lq_step_workers(Gs, Ee, Qe, W.LQ_ALPHA, W.LQ_BITS, ctx=ectx)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        og = g.lq_step_workers(Gs, Eg, Qg, W.LQ_ALPHA, W.LQ_BITS, out=og, ctx=gctx)
    torch.cuda.synchronize()
    for rep in range(4):
        for G in Gs:
            G.mul_(-1.25)                      # new gradients every step, eagerly
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe = g.lq_step_workers(Gs, Ee, Qe, W.LQ_ALPHA, W.LQ_BITS, out=oe, ctx=ectx)
        torch.cuda.synchronize()
        for k in ("p_codes", "q_codes", "p_colmax", "q_colmax", "G_hat"):
            assert torch.equal(og[k], oe[k]), "replay %d: %s" % (rep, k)
        for w in range(K):
            assert torch.equal(Eg[w], Ee[w]), "replay %d: E %d" % (rep, w)
            assert torch.equal(Qg[w], Qe[w]), "replay %d: Q %d" % (rep, w)
    del graph
    gctx.close()
    ectx.close()


def test_two_contexts_on_two_streams():
    """Each context owns its scratch: two contexts driving two streams at once (default
    priority) give the same results as one after the other."""
    g = gq()
    say("two streams")
    w = W.reduced("flat-1.3G-f32-K8-uniform127")
    xa = [x.to("cuda") for x in W.gradients(w, "cpu")]
    xb = [(-2.0 * x).contiguous() for x in xa]
    ca, cb = g.Context(), g.Context()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {}
    torch.cuda.synchronize()
    for _ in range(3):
        for name, xs, ctx, st in (("a", xa, ca, sa), ("b", xb, cb, sb)):
            with torch.cuda.stream(st):
                S, _ = g.global_norm(xs, ctx=ctx)
                outs[name] = g.fused_mean(xs, S, w.grid, w.levels, w.bits, 3, w.acc_bits, ctx=ctx)
    torch.cuda.synchronize()
    for name, xs in (("a", xa), ("b", xb)):
        S, _ = g.global_norm(xs)
        ref = g.fused_mean(xs, S, w.grid, w.levels, w.bits, 3, w.acc_bits)
        torch.cuda.synchronize()
        assert torch.equal(outs[name], ref), name
    ca.close()
    cb.close()


def test_baselines_in_a_graph(orc):
    """Per-worker scales, the per-worker-scale mean and the receiver's decode of the codes,
    captured once and replayed on new gradients: every replay equals the eager calls."""
    g = gq()
    say("graph: baselines")
    w = W.reduced("resnet50-161t-f32-K8-exp7")
    xs = [x.to("cuda") for x in W.gradients(w, "cpu")]
    gctx, ectx = g.Context(), g.Context()
    K, n = w.K, w.n
    Sg = torch.empty(K, w.nseg, dtype=torch.float32, device="cuda")
    Se = torch.empty_like(Sg)
    outs = {c: torch.empty(n, dtype=torch.float32, device="cuda") for c in ("mg", "me", "dg", "de")}
    codes_g = [torch.empty((n + 1) // 2, dtype=torch.uint8, device="cuda") for _ in range(K)]
    codes_e = [torch.empty_like(c) for c in codes_g]
    assert (w.nseg * 4) % 16 == 0  # each worker's row of scales is itself 16-byte aligned

    def step(ctx, S, m_out, d_out, codes):
        g.worker_scales(xs, g.NORM_L2, w.offsets, out=S, ctx=ctx)
        g.worker_mean(xs, S, w.grid, w.levels, 5, 0, offsets=w.offsets, out=m_out, ctx=ctx)
        for k in range(K):
            g.quantize_pack(xs[k], S[k], w.grid, w.levels, w.bits, 5, k, 0, w.offsets,
                            codes=codes[k], ctx=ctx)
        g.decode_workers(codes, n, S, w.grid, w.levels, w.bits, 0, w.offsets, out=d_out,
                         ctx=ctx)

    step(gctx, Sg, outs["mg"], outs["dg"], codes_g)   # sizes the scratch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gctx, Sg, outs["mg"], outs["dg"], codes_g)
    for rep in range(3):
        for x in xs:
            x.mul_(-1.5 if rep % 2 == 0 else 0.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(ectx, Se, outs["me"], outs["de"], codes_e)
        torch.cuda.synchronize()
        assert torch.equal(Sg, Se), "replay %d: scales" % rep
        assert torch.equal(outs["mg"], outs["me"]), "replay %d: mean" % rep
        assert torch.equal(outs["dg"], outs["de"]), "replay %d: decode" % rep
        assert torch.equal(outs["dg"], outs["mg"]), "replay %d: decode vs mean" % rep
    ref = orc.worker_mean([host(x) for x in xs], host(Se), w.grid, w.levels, 5,
                          offsets=w.offsets)
    assert np.array_equal(host(outs["mg"]), ref), first_diff(host(outs["mg"]), ref)
    del graph
    gctx.close()
    ectx.close()



def test_default_context_warm_up_then_capture(orc):
    """The default context: calls made eagerly first can then be captured on torch's capture
    stream without allocating, and the replays equal the eager results."""
    g = gq()
    say("graph: default context")
    w = W.reduced("gpt2s-148t-bf16-K16-uniform7")
    xs = [x.to("cuda") for x in W.gradients(w, "cpu")]
    S = torch.empty(w.nseg, dtype=torch.float32, device="cuda")
    out = torch.empty(w.n, dtype=torch.bfloat16, device="cuda")

    def step():
        g.global_norm(xs, w.offsets, scale_out=S)
        g.fused_mean(xs, S, w.grid, w.levels, w.bits, 2, w.acc_bits, 1, offsets=w.offsets,
                     out=out)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(2):
        for x in xs:
            x.mul_(2.0 if rep == 0 else -0.25)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got, out), "replay %d" % rep
    ref = orc.allreduce_mean([host(x) for x in xs], w.grid, w.levels, w.bits, w.acc_bits, 2, 0,
                             w.offsets, out_dtype=1, scale=host(S))
    assert np.array_equal(host(out), ref["mean"]), first_diff(host(out), ref["mean"])
    del graph


def test_replay_after_scratch_growth_and_table_eviction(orc):
    """A graph keeps the scratch and segment table of the calls it captured.  Later eager calls
    on the same context that grow its scratch (a much longer buffer) and evict its cached
    layouts (65 new ones) retire those buffers instead of freeing them, so the replays still
    match the eager calls; gq_trim then frees what was retired and eager calls go on."""
    g = gq()
    say("graph: replay after growth and eviction")
    w = W.reduced("resnet50-161t-f32-K8-exp7")
    xs = [x.to("cuda") for x in W.gradients(w, "cpu")]
    gctx, ectx = g.Context(), g.Context()
    S = torch.empty(w.nseg, dtype=torch.float32, device="cuda")
    out = torch.empty(w.n, dtype=torch.float32, device="cuda")

    def step(ctx, S_, out_):
        g.global_norm(xs, w.offsets, scale_out=S_, ctx=ctx)
        g.fused_mean(xs, S_, w.grid, w.levels, w.bits, 5, w.acc_bits, 0, offsets=w.offsets,
                     out=out_, ctx=ctx)

    step(gctx, S, out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gctx, S, out)
    torch.cuda.synchronize()
    # grow the norm scratch: 8 workers of 2^26 elements need far more tile partials
    big = [torch.randn(1 << 26, device="cuda") for _ in range(8)]
    g.global_norm(big, None, ctx=gctx)
    # evict the cached layouts: 65 distinct two-segment layouts
    y = torch.randn(65 * 8 + 64, device="cuda")
    s1 = torch.ones(2, dtype=torch.float32, device="cuda")
    for t in range(65):
        g.quantize_pack(y, s1, 0, 7, 8, 1, 0, offsets=[0, 8 * (t + 1), y.numel()], ctx=gctx)
    torch.cuda.synchronize()
    del big
    S_e, out_e = torch.empty_like(S), torch.empty_like(out)
    for rep in range(3):
        for x in xs:
            x.mul_(-1.25)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(ectx, S_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(S, S_e), "replay %d: scale" % rep
        assert torch.equal(out, out_e), "replay %d: %s" % (rep, first_diff(host(out), host(out_e)))
    ref = orc.allreduce_mean([host(x) for x in xs], w.grid, w.levels, w.bits, w.acc_bits, 5, 0,
                             w.offsets, scale=host(S))
    assert np.array_equal(host(out), ref["mean"]), first_diff(host(out), ref["mean"])
    del graph
    g.trim(ctx=gctx)
    step(gctx, S, out)
    torch.cuda.synchronize()
    assert torch.equal(out, out_e)
    gctx.close()
    ectx.close()


def test_lq_replay_after_scratch_growth():
    """The LQ-SGD step captured on a context whose scratch a larger eager step then replaces:
    the replays still equal the eager step on a second context bit for bit."""
    g = gq()
    n, m, r = 512, 384, 3
    say("graph: lq replay after growth", n, m, r)
    gen = torch.Generator(device="cuda").manual_seed(23)
    G = torch.randn(n, m, device="cuda", generator=gen) * 1e-3
    E0 = torch.randn(n, m, device="cuda", generator=gen) * 1e-4
    Q0 = torch.randn(m, r, device="cuda", generator=gen)
    gctx, ectx = g.Context(), g.Context()
    Eg, Qg, Ee, Qe = E0.clone(), Q0.clone(), E0.clone(), Q0.clone()
    og = g.powersgd_logquant(G, Eg, Qg, W.LQ_ALPHA, W.LQ_BITS, ctx=gctx)
    oe = g.powersgd_logquant(G, Ee, Qe, W.LQ_ALPHA, W.LQ_BITS, ctx=ectx)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        og = g.powersgd_logquant(G, Eg, Qg, W.LQ_ALPHA, W.LQ_BITS, out=og, ctx=gctx)
    torch.cuda.synchronize()
    # a much larger step on the capturing context replaces its scratch
    Gb = torch.randn(4096, 4096, device="cuda", generator=gen)
    g.powersgd_logquant(Gb, torch.zeros_like(Gb), torch.randn(4096, 8, device="cuda",
                                                              generator=gen),
                        W.LQ_ALPHA, W.LQ_BITS, ctx=gctx)
    torch.cuda.synchronize()
    del Gb
    for rep in range(3):
        G.mul_(-1.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe = g.powersgd_logquant(G, Ee, Qe, W.LQ_ALPHA, W.LQ_BITS, out=oe, ctx=ectx)
        torch.cuda.synchronize()
        for k in ("p_codes", "q_codes", "p_colmax", "q_colmax", "p_hat"):
            assert torch.equal(og[k], oe[k]), "replay %d: %s" % (rep, k)
        assert torch.equal(Eg, Ee) and torch.equal(Qg, Qe), "replay %d" % rep
    del graph
    g.trim(ctx=gctx)
    gctx.close()
    ectx.close()
