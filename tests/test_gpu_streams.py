"""Streams and graphs.  The library enqueues only on its context's stream
and allocates nothing per call, so a context can run on a side stream, two
contexts can run on two streams at once, and a whole step (the L1 path's
three kernels, or the vote kernel) can be captured into a HIP graph and
replayed.  Every result is compared with the CPU oracle bit for bit."""
import numpy as np
import pytest

from oracle import lco
from synth import gen
from synth import workloads as wls
from tests.harness import check_float_state, lioncub_for, to_dev, to_host

pytestmark = pytest.mark.gpu


def _host_state(wl):
    return gen.host_theta(wl), gen.host_m(wl)


def _check(wl, d_theta, d_m, theta, m, what):
    check_float_state(f"theta {what}", to_host(d_theta), theta, bf16=wl.theta_dtype == "bf16")
    check_float_state(f"m {what}", to_host(d_m)[:, : wl.d], m[:, : wl.d])


def test_context_on_a_side_stream():
    import torch
    wl = wls.flat("ss", 3 * 4096 + 100, W=8, agg="l1", qbits=4)
    theta, m = _host_state(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lc = lioncub_for(wl, stream=s)
        d_theta, d_m = to_dev(theta), to_dev(m)
        for t in (1, 2):
            g = gen.host_g(wl, t)
            lc.step(d_theta, d_m, to_dev(g), t)
            lco.step(wl, theta, m, g, t)
    s.synchronize()
    _check(wl, d_theta, d_m, theta, m, "side stream")
    lc.close()


def test_two_contexts_on_two_streams_at_once():
    import torch
    wa = wls.flat("sa", 4 * 4096 + 64, W=4, theta_dtype="bf16", grad_dtype="bf16")
    wb = wls.Workload(name="sb", tensors=[("x", 2 * 4096 + 320), ("y", 4096)], W=16, agg="l1",
                      qbits=4)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ha, hb = _host_state(wa), _host_state(wb)
    ga = [gen.host_g(wa, t) for t in (1, 2, 3)]
    gb = [gen.host_g(wb, t) for t in (1, 2, 3)]
    da = (to_dev(ha[0], True), to_dev(ha[1]), [to_dev(x, True) for x in ga])
    db = (to_dev(hb[0]), to_dev(hb[1]), [to_dev(x) for x in gb])
    torch.cuda.synchronize()
    la, lb = lioncub_for(wa, stream=sa), lioncub_for(wb, stream=sb)
    for k, t in enumerate((1, 2, 3)):          # interleaved launches on two streams
        with torch.cuda.stream(sa):
            la.step(da[0], da[1], da[2][k], t)
        with torch.cuda.stream(sb):
            lb.step(db[0], db[1], db[2][k], t)
    torch.cuda.synchronize()
    for k, t in enumerate((1, 2, 3)):
        lco.step(wa, ha[0], ha[1], ga[k], t)
        lco.step(wb, hb[0], hb[1], gb[k], t)
    _check(wa, da[0], da[1], ha[0], ha[1], "stream a")
    _check(wb, db[0], db[1], hb[0], hb[1], "stream b")
    la.close()
    lb.close()


@pytest.mark.parametrize("agg", ["vote", "l1", "linf"])
def test_step_captured_in_a_graph_and_replayed(agg):
    """Capture one step at a fixed t, replay it three times with eager steps
    of another context and host synchronisations in between; every replay
    must equal the oracle's step from the previous state."""
    import torch
    wl = wls.Workload(name="gr", tensors=[("a", 5 * 4096 + 192), ("b", 4096 + 64)], W=8,
                      agg=agg, qbits=0 if agg == "vote" else 4, sync_names=("b",),
                      sync_every=3)
    theta, m = _host_state(wl)
    g = gen.host_g(wl, 3)
    t = 3                                      # an averaging step for tensor b
    d_theta, d_m, d_g = to_dev(theta), to_dev(m), to_dev(g)
    lc = lioncub_for(wl)
    # eager side work: a second context stepping its own copy of the state
    e_theta, e_m = to_dev(theta), to_dev(m)
    le = lioncub_for(wl)
    h_theta, h_m = theta.copy(), m.copy()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lc.set_stream(torch.cuda.current_stream())
        lc.step(d_theta, d_m, d_g, t)
    lc.set_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    _check(wl, d_theta, d_m, theta, m, "after capture (nothing ran)")

    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        lco.step(wl, theta, m, g, t)
        _check(wl, d_theta, d_m, theta, m, f"replay {rep}")
        le.step(e_theta, e_m, d_g, t)          # eager work between replays
        torch.cuda.synchronize()
        lco.step(wl, h_theta, h_m, g, t)
        _check(wl, e_theta, e_m, h_theta, h_m, f"eager {rep}")
    del graph
    lc.close()
    le.close()


def test_two_contexts_from_two_host_threads():
    """The library keeps no global state: two host threads, each with its own
    context and stream, step concurrently (ctypes releases the GIL during
    the calls); both results equal the oracle's."""
    import threading

    import torch
    wls_ = [wls.flat("ta", 3 * 4096 + 192, W=8, agg="l1", qbits=4),
            wls.flat("tb", 5 * 4096 + 64, W=5, agg="vote", tie="zero", grad_dtype="bf16")]
    results = [None, None]
    errors = []

    def worker(k):
        try:
            wl = wls_[k]
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            theta, m = _host_state(wl)
            gs = [gen.host_g(wl, t) for t in (1, 2, 3, 4)]
            with torch.cuda.stream(s):
                lc = lioncub_for(wl, stream=s)
                d_theta, d_m = to_dev(theta), to_dev(m)
                d_gs = [to_dev(g, wl.grad_dtype == "bf16") for g in gs]
                for t in (1, 2, 3, 4):
                    lc.step(d_theta, d_m, d_gs[t - 1], t)
            s.synchronize()
            for t in (1, 2, 3, 4):
                lco.step(wl, theta, m, gs[t - 1], t)
            results[k] = (wl, d_theta, d_m, theta, m)
            lc.close()
        except Exception as e:  # reported below
            errors.append(repr(e))

    th = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors, errors
    for wl, d_theta, d_m, theta, m in results:
        _check(wl, d_theta, d_m, theta, m, f"thread {wl.name}")


@pytest.mark.parametrize("agg,sync_every,K", [("vote", 1, 2), ("l1", 3, 6), ("avg", 2, 4)])
def test_captured_window_replays_as_the_next_steps(agg, sync_every, K):
    """LionCub.capture: a window of K steps (K a multiple of lcm(2,
    sync_every)) replayed three times equals 3K consecutive eager steps of
    the oracle, with the gradients refilled between replays."""
    import torch
    wl = wls.Workload(name="cw", tensors=[("a", 2 * 4096 + 192), ("b", 4096 + 64)], W=4,
                      agg=agg, qbits=4 if agg == "l1" else 0, sync_names=("b",),
                      sync_every=sync_every)
    theta, m = _host_state(wl)
    d_theta, d_m = to_dev(theta), to_dev(m)
    d_gs = [torch.empty((wl.W, wl.ld), device="cuda") for _ in range(K)]
    lc = lioncub_for(wl)
    t0 = 5
    graph = lc.capture(d_theta, d_m, d_gs, t0)
    torch.cuda.synchronize()
    _check(wl, d_theta, d_m, theta, m, "after capture (nothing ran)")
    t = t0
    for rep in range(3):
        gs = [gen.host_g(wl, t + k) for k in range(K)]
        for k in range(K):
            d_gs[k].copy_(to_dev(gs[k]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in range(K):
            lco.step(wl, theta, m, gs[k], t + k)
        _check(wl, d_theta, d_m, theta, m, f"replay {rep}")
        t += K
    del graph
    lc.close()


def test_capture_refuses_windows_that_would_not_replay_exactly():
    import torch
    wl = wls.flat("cr", 4096, W=2, agg="vote", sync_every=3)
    lc = lioncub_for(wl)
    th, m = to_dev(_host_state(wl)[0]), to_dev(_host_state(wl)[1])
    gs = [torch.zeros((2, wl.ld), device="cuda") for _ in range(4)]
    with pytest.raises(ValueError):
        lc.capture(th, m, gs, 1)                    # 4 is not a multiple of lcm(2, 3) = 6
    lc.profile_begin(8)
    with pytest.raises(ValueError):
        lc.capture(th, m, gs[:2] * 3, 1)            # profiling events would enter the graph
    lc.profile_end()
    lc.close()
    wi = wls.flat("ci", 4096, W=2, agg="linf", qbits=4)
    li = lioncub_for(wi)
    with pytest.raises(ValueError):
        li.capture(th, m, gs[:2], 1)                # max-norm draws depend on the full t
    li.close()


def test_probe_stream_kernels():
    """The measurement library's reference kernels compute what they claim:
    copy c = a, triad c = a + 0.5 b (0.5 b is exact, so one rounding)."""
    import torch

    from communication_compressed_distributed_amd import _abi, _probe
    n = 3 * 4096
    rs = np.random.default_rng(2)
    a_h = rs.normal(0, 1, n).astype(np.float32)
    b_h = rs.normal(0, 1, n).astype(np.float32)
    a, b = to_dev(a_h), to_dev(b_h)
    c = torch.full((n,), 7.0, device="cuda")
    h = _abi._stream_handle()
    _probe.lioncub_probe_stream(_probe.PROBE_READ, a, None, c, n, h)
    torch.cuda.synchronize()
    assert torch.all(c == 7.0)                 # the read kernel writes nothing
    _probe.lioncub_probe_stream(_probe.PROBE_COPY, a, None, c, n, h)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(c), a_h)
    _probe.lioncub_probe_stream(_probe.PROBE_TRIAD, a, b, c, n, h)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(c), a_h + np.float32(0.5) * b_h)


def test_probe_step_pattern_touches_every_element():
    """The step-pattern probe reads and writes exactly the step's elements:
    every worker's m becomes beta2*m + (1-beta2)*g (one rounding each, no
    contraction), columns past d stay, and every theta moves by +-lr."""
    import torch

    from communication_compressed_distributed_amd import _abi, _probe
    rs = np.random.default_rng(3)
    for W, d, gd, flags in ((16, 5 * 4096 + 900, 0, 0), (5, 4096 + 64, 1, 0), (8, 3 * 4096, 1, 1),
                            (4, 2 * 4096 + 36, 0, 1), (16, 3 * 4096 + 100, 0, 2), (5, 2 * 4096, 1, 3),
                            (16, 3 * 4096 + 64, 0, 4), (3, 2 * 4096 + 8, 1, 8), (8, 4096, 0, 12),
                            (7, 3 * 4096 + 4, 0, 16), (16, 2 * 4096 + 12, 1, 32),
                            (2, 4 * 4096 + 2000, 0, 48)):
        ld = (d + 63) // 64 * 64 + 64
        th_h = rs.normal(0, 0.02, d).astype(np.float32)
        m_h = rs.normal(0, 1e-3, (W, ld)).astype(np.float32)
        g32 = rs.normal(0, 1e-3, (W, ld)).astype(np.float32)
        th, m = to_dev(th_h), to_dev(m_h)
        if gd:
            g = torch.from_numpy(g32).to(torch.bfloat16).cuda()
            gw = g.float().cpu().numpy()
        else:
            g = to_dev(g32)
            gw = g32
        beta2, lr = np.float32(0.99), np.float32(1e-4)
        _probe.lioncub_probe_step_pattern(th, m, g, d, ld, W, 0, gd, float(beta2), float(lr),
                                          _abi._stream_handle(), flags=flags)
        torch.cuda.synchronize()
        want = (beta2 * m_h[:, :d]) + ((np.float32(1) - beta2) * gw[:, :d])
        got = to_host(m)
        assert np.array_equal(got[:, :d], want)
        assert np.array_equal(got[:, d:], m_h[:, d:])
        moved = to_host(th) - th_h
        assert np.all((moved != 0))


def test_probe_panel_pattern_touches_every_element():
    """The panel-arrangement probe also reads and writes every element of
    every worker exactly once (m <- beta2*m + (1-beta2)*g), whatever the
    panel width, including a short last panel and a ragged last block."""
    import torch

    from communication_compressed_distributed_amd import _abi, _probe
    rs = np.random.default_rng(4)
    for W, d, panel in ((16, 5 * 4096 + 900, 2), (3, 7 * 4096, 4), (8, 2 * 4096 + 64, 64)):
        ld = (d + 63) // 64 * 64
        th_h = rs.normal(0, 0.02, d).astype(np.float32)
        m_h = rs.normal(0, 1e-3, (W, ld)).astype(np.float32)
        g_h = rs.normal(0, 1e-3, (W, ld)).astype(np.float32)
        th, m, g = to_dev(th_h), to_dev(m_h), to_dev(g_h)
        beta2 = np.float32(0.99)
        _probe.lioncub_probe_panel_pattern(th, m, g, d, ld, W, 0, 0, float(beta2), 1e-4, panel,
                                           _abi._stream_handle())
        torch.cuda.synchronize()
        want = (beta2 * m_h[:, :d]) + ((np.float32(1) - beta2) * g_h[:, :d])
        assert np.array_equal(to_host(m)[:, :d], want)
        assert np.all(to_host(th) != th_h)
