"""Full-size parity: the five workloads at their real sizes, run with the
production kernels bench.py times, checked against the CPU oracle on sampled
column ranges (first, last -- the ragged end --, tensor boundaries and random
interior ranges).  On the L1 workloads the oracle first recomputes M1 from
the pre-step state, streamed from the device one worker row at a time, for
every (worker, tensor) pair the samples touch (all of them for the flat 350M
model), and M1 itself is compared bit for bit with the library's.  The
max-norm baseline on the flat 350M shape does the same with max |c|."""
import numpy as np
import pytest

from oracle import lco
from synth import gen
from synth import workloads as wls
from tests.harness import check_float_state, lioncub_for, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

STREAM = 1 << 24  # elements per host round trip when recomputing M1


def _say(*a):
    print("[fullsize]", *a, flush=True)


def sample_ranges(wl, tensors, rs, width=65536, n_random=6):
    """Column ranges inside the given tensors: each tensor's start, its end
    and one random interior range (all within the tensor)."""
    out = []
    off = wl.offsets
    for T in tensors:
        a, b = off[T], off[T + 1]
        w = min(width, b - a)
        out.append((a, a + w))
        out.append((b - w, b))
        for _ in range(n_random):
            if b - a > 2 * w:
                s = int(rs.integers(a, b - w)) // 64 * 64
                out.append((s, s + w))
    return sorted(set(out))


def oracle_m1(wl, m, g, pairs):
    """M1[i][T] for the requested (worker, tensor) pairs from device state."""
    off = wl.offsets
    res = {}
    for (i, T) in pairs:
        a, b = off[T], off[T + 1]
        parts = []
        for s in range(a, b, STREAM):
            e = min(b, s + STREAM)
            parts.append(lco.m1_partials(wl, to_host(m[i, s:e]), to_host(g[i, s:e])))
        res[(i, T)] = lco.m1_finalize(np.concatenate(parts), b - a)
    return res


def oracle_minf(wl, m, g, pairs):
    """max |c|[i][T] for the requested pairs (a maximum: chunk order is free)."""
    off = wl.offsets
    res = {}
    for (i, T) in pairs:
        a, b = off[T], off[T + 1]
        v = 0.0
        for s in range(a, b, STREAM):
            e = min(b, s + STREAM)
            v = max(v, lco.minf(lco.c_row(wl, to_host(m[i, s:e]), to_host(g[i, s:e]))))
        res[(i, T)] = v
    return res


def run_fullsize(wl, steps, tensors=None, n_random=6):
    import torch
    torch.cuda.set_device(0)
    rs = np.random.default_rng(7)
    tensors = list(range(wl.n_tensors)) if tensors is None else tensors
    ranges = sample_ranges(wl, tensors, rs, n_random=n_random)
    _say(wl.name, f"d={wl.d} W={wl.W} ranges={len(ranges)} tensors={len(tensors)}")
    theta = gen.device_theta(wl)
    m = gen.device_m(wl)
    g = gen.device_g(wl, steps[0])
    lc = lioncub_for(wl)
    tb = wl.theta_dtype == "bf16"
    for t in steps:
        gen.fill_device_g(wl, t, g)
        torch.cuda.synchronize()
        pre = [(j0, j1, to_host(theta[j0:j1]).copy(), to_host(m[:, j0:j1]).copy(),
                to_host(g[:, j0:j1]).copy()) for j0, j1 in ranges]
        m1v = None
        dbg = None
        if wl.agg in ("l1", "linf"):
            pairs = [(i, T) for i in range(wl.W) for T in tensors]
            want_m1 = (oracle_m1 if wl.agg == "l1" else oracle_minf)(wl, m, g, pairs)
            _say(wl.name, f"t={t} oracle M1 done for {len(pairs)} pairs")
            m1v = np.full((wl.W, wl.n_tensors), np.nan)
            for (i, T), v in want_m1.items():
                m1v[i, T] = v
            dbg = {"m1": torch.zeros((wl.W, wl.n_tensors), dtype=torch.float64, device="cuda")}
        lc.step(theta, m, g, t, dbg)
        torch.cuda.synchronize()
        if dbg is not None:
            got = to_host(dbg["m1"])
            for (i, T), v in want_m1.items():
                assert np.float64(got[i, T]).view(np.uint64) == np.float64(v).view(np.uint64), \
                    (i, T, got[i, T], v)
        for j0, j1, th, mc, gc in pre:
            mc = np.ascontiguousarray(mc)
            lco.step_range(wl, j0, j1, m1v, th, mc, np.ascontiguousarray(gc), t)
            check_float_state(f"theta[{j0}:{j1}] t={t}", to_host(theta[j0:j1]), th, bf16=tb)
            check_float_state(f"m[:, {j0}:{j1}] t={t}", to_host(m[:, j0:j1]), mc)
        _say(wl.name, f"t={t} ok")
    lc.close()
    del theta, m, g
    torch.cuda.empty_cache()


def run_every_element(wl, steps):
    """The workload at its real size for its steps, every element of theta
    and m (and every norm) compared with the oracle after every step.  The
    oracle steps from the device's pre-step snapshot and the device state is
    never reset; with every step required bit-equal, the device's trajectory
    is the oracle's (test_independent_trajectory_at_full_size runs the two
    apart on the workloads whose state fits in host memory)."""
    import torch
    from tests.fullsize_check import check_step_every_element
    torch.cuda.set_device(0)
    _say(wl.name, f"every element: d={wl.d} W={wl.W} steps={steps}")
    theta = gen.device_theta(wl)
    m = gen.device_m(wl)
    g = gen.device_g(wl, steps[0])
    lc = lioncub_for(wl)
    for t in steps:
        gen.fill_device_g(wl, t, g)
        torch.cuda.synchronize()
        check_step_every_element(wl, lc, theta, m, g, t)
    lc.close()
    del theta, m, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl", wls.ALL, ids=lambda w: w.name)
def test_every_element_at_full_size(wl):
    """All five workloads at their full shapes and step counts (10, 5, 5, 3
    and 3 steps): every parameter, every momentum of every worker, and on
    the L1 workloads the mean |c| of every (worker, tensor) pair."""
    run_every_element(wl, list(range(1, wl.steps + 1)))


def _oracle_step_threaded(wl, theta, m, g, t, P=16):
    """One oracle step (vote or averaging path: no norms) on host arrays in
    place, its columns split over P threads on disjoint 64-aligned ranges
    (a column's update reads and writes nothing outside it)."""
    import ctypes as C
    from concurrent.futures import ThreadPoolExecutor
    L = lco.lib()
    cfg = lco.OracleCfg(wl)
    ld = m.shape[1]
    per = (-(-wl.d // P) + 63) // 64 * 64
    ranges = [(a, min(wl.d, a + per)) for a in range(0, wl.d, per)]

    def run(r):
        a, b = r
        L.lco_step_range(cfg.ref, a, b, None, C.c_void_p(theta.ctypes.data + a * theta.itemsize),
                         C.c_void_p(m.ctypes.data + a * m.itemsize),
                         C.c_void_p(g.ctypes.data + a * g.itemsize), ld, t, None)
    with ThreadPoolExecutor(P) as pool:
        list(pool.map(run, ranges))


@pytest.mark.parametrize("wl", [wls.FLAT_1M_W4_VOTE, wls.GPT2_124M_W8_VOTE], ids=lambda w: w.name)
def test_independent_trajectory_at_full_size(wl):
    """The 1M x 4 workload over its 10 steps and the GPT-2 small list
    (124M x 8) over its 5, each side carrying its own theta and m from the
    same seeded start: the oracle on host copies, the library on the device,
    nothing passed from one to the other but each step's gradients.  Every
    element is compared after every step and at the end."""
    import torch
    torch.cuda.set_device(0)
    theta = gen.device_theta(wl)
    m = gen.device_m(wl)
    g = gen.device_g(wl, 1)
    th_h, m_h = to_host(theta).copy(), to_host(m).copy()
    lc = lioncub_for(wl)
    tb = wl.theta_dtype == "bf16"
    for t in range(1, wl.steps + 1):
        gen.fill_device_g(wl, t, g)
        torch.cuda.synchronize()
        g_h = to_host(g)
        lc.step(theta, m, g, t)
        _oracle_step_threaded(wl, th_h, m_h, g_h, t)
        torch.cuda.synchronize()
        for name, got, want in ((f"theta t={t}", to_host(theta), th_h),
                                (f"m t={t}", to_host(m)[:, : wl.d], m_h[:, : wl.d])):
            u = np.uint16 if tb and name.startswith("theta") else np.uint32
            if not np.array_equal(got.view(u), want.view(u)):     # the full bar says what differs
                check_float_state(name, got, want, bf16=(u == np.uint16))
        _say(wl.name, f"independent trajectories equal after step {t}")
    lc.close()
    del theta, m, g
    torch.cuda.empty_cache()


EXTRA_EVERY_ELEMENT = {
    # the max-norm stochastic baseline at the flat 350M x 16 shape (n = 4):
    # its draws depend on t, d, W, i and j, so every element is its own case
    "flat-350M-w16-linfq4": wls.FLAT_350M_W16_L1Q4.with_(name="flat-350M-w16-linfq4",
                                                         agg="linf", steps=3),
    # D-Lion averaging (fractional update (2v - W)/W) on the GPT-2 small list
    "gpt2-124M-w8-avg": wls.GPT2_124M_W8_VOTE.with_(name="gpt2-124M-w8-avg", agg="avg"),
    # the 2-bit-result vote (ties give 0) on the 760M list with averaging
    # every other step
    "gpt-760M-w8-tiezero-sync2": wls.GPT_760M_W8_VOTE_SYNC.with_(
        name="gpt-760M-w8-tiezero-sync2", tie="zero", sync_every=2, steps=2),
}


@pytest.mark.parametrize("name", list(EXTRA_EVERY_ELEMENT))
def test_every_element_other_aggregations(name):
    """The other aggregation modes at full size, every element and every
    norm compared after every step."""
    wl = EXTRA_EVERY_ELEMENT[name]
    run_every_element(wl, list(range(1, wl.steps + 1)))


def test_flat_1M_w4_vote_fullsize():
    run_fullsize(wls.FLAT_1M_W4_VOTE, steps=list(range(1, 11)))


def test_gpt2_124M_w8_vote_fullsize():
    wl = wls.GPT2_124M_W8_VOTE
    run_fullsize(wl, steps=[1, 2], n_random=1)


def test_flat_350M_w16_l1q4_fullsize():
    run_fullsize(wls.FLAT_350M_W16_L1Q4, steps=[1, 2])


def test_flat_350M_w16_linfq4_fullsize():
    """The max-norm baseline at the flat 350M, W=16, n=4 shape."""
    wl = wls.FLAT_350M_W16_L1Q4.with_(name="flat-350M-w16-linfq4", agg="linf")
    run_fullsize(wl, steps=[3])


def test_gpt_760M_w8_vote_bf16_sync_fullsize():
    wl = wls.GPT_760M_W8_VOTE_SYNC
    run_fullsize(wl, steps=[1, 2, 3], n_random=1)


def test_gpt_1B3_w8_l1q8_bf16g_fullsize():
    """M1 recomputed on the host for the embeddings, the first and last
    transformer blocks and the final LayerNorm (the samples' tensors)."""
    wl = wls.GPT_1B3_W8_L1Q8
    names = [nm for nm, _ in wl.tensors]
    pick = [k for k, nm in enumerate(names)
            if nm in ("wte", "wpe", "ln_f.w", "ln_f.b") or nm.startswith(("h0.", "h23."))]
    run_fullsize(wl, steps=[1, 2], tensors=pick, n_random=1)


@pytest.mark.parametrize("agg", ["vote", "l1"])
def test_beyond_two_to_the_31_elements(agg):
    """A vector of 2^31 + 4160 elements (2 workers): every element index,
    block index and word index past 2^31 must be 64-bit; the samples include
    the ragged end, and on the L1 path M1 of both rows is recomputed on the
    host and compared bit for bit."""
    wl = wls.flat(f"flat-2G-w2-{agg}", 2**31 + 4160, W=2, agg=agg, qbits=4 if agg == "l1" else 0,
                  g_nu=3.0)
    run_fullsize(wl, steps=[1], n_random=2)


def test_pack_and_vote_beyond_two_to_the_31_elements():
    """lioncub_pack and lioncub_vote_bits on 3 rows of 2^31 + 4160 elements:
    sampled word ranges (first, around 2^31, last) against the oracle."""
    import torch
    torch.cuda.set_device(0)
    wl = wls.flat("flat-2G-w3-pack", 2**31 + 4160, W=3)
    lc = lioncub_for(wl)
    x = gen.device_m(wl)                          # any fp32 rows stand in for c
    x[:, ::4099] = 0.0                            # exact zeros: the parity rule
    words = wl.ld // 64
    bits = torch.empty((wl.W, words), dtype=torch.int64, device="cuda")
    sign_p = torch.empty(words, dtype=torch.int64, device="cuda")
    zero_p = torch.empty(words, dtype=torch.int64, device="cuda")   # 16-byte aligned each
    t = 3
    lc.pack(x, t, bits)
    lc.vote_bits(bits, t, sign_p, zero_p)
    torch.cuda.synchronize()
    for w0 in (0, (2**31 // 64) - 512, words - 1024):
        w1 = min(words, w0 + 1024)
        j0, j1 = 64 * w0, min(wl.d, 64 * w1)
        xs = np.zeros((wl.W, 64 * (w1 - w0)), np.float32)
        xs[:, : j1 - j0] = to_host(x[:, j0:j1])
        want = lco.pack(xs, j1 - j0, t)
        got = to_host(bits[:, w0:w1]).view(np.uint64)
        assert np.array_equal(got, want), (w0, w1)
        sb, zb = lco.vote_bits(want, wl.W, j1 - j0, t)
        assert np.array_equal(to_host(sign_p[w0:w1]).view(np.uint64), sb), (w0, w1)
        _say("pack/vote_bits words", w0, w1, "ok")
    lc.close()
    del x, bits, sign_p, zero_p
    torch.cuda.empty_cache()


def test_entry_points_at_bench_size():
    """Every standalone entry point on the 350M x 16 shape the benchmark
    times with --op (same launch configuration): pack, vote (counts, signs
    and bit planes), quant_l1 and quant_linf (the per-row norms of all 16
    rows recomputed on the host and compared bit for bit; codes on sampled
    columns), pack_codes and unpack_sum, and apply from the voted planes, each
    checked against the oracle on the first columns, an interior range and
    the last columns (unpack_sum_bits too)."""
    import torch
    torch.cuda.set_device(0)
    wl = wls.FLAT_350M_W16_L1Q4
    W, d, ld, n = wl.W, wl.d, wl.ld, wl.qbits
    t = 3
    lc = lioncub_for(wl)
    x = gen.device_g(wl, 1)                        # heavy-tailed fp32 rows stand in for c
    x[:, ::4099] = 0.0                             # exact zeros: the parity rule
    words = ld // 64
    bits = torch.empty((W, words), dtype=torch.int64, device="cuda")
    counts = torch.empty(d, dtype=torch.uint8, device="cuda")
    sign = torch.empty(d, dtype=torch.int8, device="cuda")
    sign_p = torch.empty(words, dtype=torch.int64, device="cuda")
    zero_p = torch.empty(words, dtype=torch.int64, device="cuda")
    codes = torch.empty((W, ld), dtype=torch.int8, device="cuda")
    codes_inf = torch.empty((W, ld), dtype=torch.int8, device="cuda")
    m1 = torch.empty((W, 1), dtype=torch.float64, device="cuda")
    minf = torch.empty((W, 1), dtype=torch.float64, device="cuda")
    wire = torch.empty((W, (ld // 32) * n), dtype=torch.int32, device="cuda")
    sums = torch.empty(d, dtype=torch.int32, device="cuda")
    usign = torch.empty(d, dtype=torch.int8, device="cuda")
    usb = torch.empty(words, dtype=torch.int64, device="cuda")
    uzb = torch.empty(words, dtype=torch.int64, device="cuda")
    lc.pack(x, t, bits)
    lc.vote(bits, t, counts, sign)
    lc.vote_bits(bits, t, sign_p, zero_p)
    lc.quant_l1(x, codes, m1)
    lc.quant_linf(x, t, codes_inf, minf)
    lc.pack_codes(codes, wire)
    lc.unpack_sum(wire, sums, usign)
    lc.unpack_sum_bits(wire, usb, uzb)
    torch.cuda.synchronize()
    _say("entry points ran on", wl.name)

    # the per-row norms of every row, from the whole row on the host
    got_m1, got_minf = to_host(m1)[:, 0], to_host(minf)[:, 0]
    for i in range(W):
        row = to_host(x[i, :d])
        assert np.float64(got_m1[i]).view(np.uint64) == np.float64(lco.m1(row)).view(np.uint64), i
        assert got_minf[i] == lco.minf(row), i
    _say("norms of", W, "rows ok")

    width = 65536
    ranges = [(0, width), ((d // 2) // 64 * 64, (d // 2) // 64 * 64 + width), (d - width, d)]
    for j0, j1 in ranges:
        w0, w1 = j0 // 64, j1 // 64
        xs = np.ascontiguousarray(to_host(x[:, j0:j1]))
        want_bits = lco.pack(xs, j1 - j0, t)
        assert np.array_equal(to_host(bits[:, w0:w1]).view(np.uint64), want_bits), (j0, "pack")
        wc, ws = lco.vote(want_bits, W, j1 - j0, t)
        assert np.array_equal(to_host(counts[j0:j1]), wc), (j0, "counts")
        assert np.array_equal(to_host(sign[j0:j1]), ws), (j0, "sign")
        sb, zb = lco.vote_bits(want_bits, W, j1 - j0, t)
        assert np.array_equal(to_host(sign_p[w0:w1]).view(np.uint64), sb), (j0, "sign planes")
        assert np.array_equal(to_host(zero_p[w0:w1]).view(np.uint64), zb), (j0, "zero planes")
        # codes, element by element on the first 2048 columns of the range
        cs = to_host(codes[:, j0:j1])
        ci = to_host(codes_inf[:, j0:j1])
        for i in range(W):
            for k in range(2048):
                j = j0 + k
                assert cs[i, k] == lco.q1(xs[i, k], got_m1[i], n), (i, j, "q1")
                r = lco.sr_u32(wl.sr_seed, d, W, t, i, j)
                assert ci[i, k] == lco.qinf(xs[i, k], got_minf[i], n, r), (i, j, "qinf")
        # wire format and the receive-side sum over the whole range
        want_wire = lco.pack_codes(cs, j1 - j0, n)
        g0, g1 = j0 // 32, j1 // 32
        got_wire = to_host(wire[:, g0 * n:g1 * n]).view(np.uint32)
        assert np.array_equal(got_wire, want_wire), (j0, "wire")
        us, ug = lco.unpack_sum(want_wire, W, j1 - j0, j1 - j0, n)
        assert np.array_equal(to_host(sums[j0:j1]), us), (j0, "sums")
        assert np.array_equal(to_host(usign[j0:j1]), ug), (j0, "unpack sign")
        ub, uz = lco.unpack_sum_bits(want_wire, W, j1 - j0, j1 - j0, n)
        assert np.array_equal(to_host(usb[w0:w1]).view(np.uint64), ub), (j0, "unpack sign plane")
        assert np.array_equal(to_host(uzb[w0:w1]).view(np.uint64), uz), (j0, "unpack zero plane")
        _say("range", j0, j1, "ok")
    del bits, counts, sign, codes, codes_inf, wire, sums, usign, usb, uzb
    torch.cuda.empty_cache()

    # apply from the voted planes: x is this step's g
    theta = gen.device_theta(wl)
    m = gen.device_m(wl)
    pre = [(j0, j1, to_host(theta[j0:j1]).copy(), np.ascontiguousarray(to_host(m[:, j0:j1])))
           for j0, j1 in ranges]
    lc.apply(theta, m, x, t, sign_p, zero_p)
    torch.cuda.synchronize()
    for j0, j1, th, mc in pre:
        sl = wl.with_(name="slice", tensors=[("flat", j1 - j0)])
        gs = np.ascontiguousarray(to_host(x[:, j0:j1]))
        lco.apply(sl, th, mc, gs, t, to_host(sign_p[j0 // 64:j1 // 64]).view(np.uint64),
                  to_host(zero_p[j0 // 64:j1 // 64]).view(np.uint64))
        check_float_state(f"theta[{j0}:{j1}] apply", to_host(theta[j0:j1]), th)
        check_float_state(f"m[:, {j0}:{j1}] apply", to_host(m[:, j0:j1]), mc)
    _say("apply ok")
    lc.close()
    del x, theta, m, sign_p, zero_p, m1, minf
    torch.cuda.empty_cache()


LARGE_W_CASES = {
    # many workers on states of ~6 GB: the fused step's generic worker loop
    # (W not 4, 8 or 16) at full scale, a tie-zero vote over three tensors
    "vote-W255": wls.flat("large-vote-W255", 3_158_037, W=255, agg="vote", g_nu=3.0),
    "avg-W40-bf16": wls.flat("large-avg-W40", 20_132_673, W=40, agg="avg", theta_dtype="bf16",
                             grad_dtype="bf16", g_nu=3.0),
    "vote-W17-tiezero-3T": wls.Workload(name="large-vote-W17",
                                        tensors=[("a", 20_000_064), ("b", 4160), ("c", 27_380_000)],
                                        W=17, agg="vote", tie="zero", theta_dtype="bf16",
                                        g_nu=3.0),
}


@pytest.mark.parametrize("name", sorted(LARGE_W_CASES))
def test_large_worker_counts(name):
    """Two production steps with many workers on multi-gigabyte states,
    against the oracle on sampled ranges."""
    run_fullsize(LARGE_W_CASES[name], steps=[1, 2], n_random=2)


@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16")])
def test_apply_large_state(dtypes):
    """lioncub_apply on a 33.5M x 8 state of two tensors with a ragged end,
    random sign and zero planes: sampled ranges bit for bit against the
    oracle, on a plain step and on an averaging step of the synced tensor."""
    import torch
    th_dt, g_dt = dtypes
    wl = wls.Workload(name="large-apply", tensors=[("a", 16_777_216), ("b", 16_777_216 + 4160)],
                      W=8, theta_dtype=th_dt, grad_dtype=g_dt, sync_names=("b",), sync_every=2,
                      g_nu=3.0)
    torch.cuda.set_device(0)
    lc = lioncub_for(wl)
    theta, m = gen.device_theta(wl), gen.device_m(wl)
    words = wl.ld // 64
    gen_t = torch.Generator(device="cuda").manual_seed(5)
    sb = torch.randint(-2 ** 62, 2 ** 62, (words,), generator=gen_t, device="cuda", dtype=torch.int64)
    zb = torch.randint(-2 ** 62, 2 ** 62, (words,), generator=gen_t, device="cuda", dtype=torch.int64)
    zb &= torch.randint(-2 ** 62, 2 ** 62, (words,), generator=gen_t, device="cuda", dtype=torch.int64)
    tail = wl.d // 64                                      # bits past d are 0
    if wl.d % 64:
        sb[tail] &= (1 << (wl.d % 64)) - 1
        zb[tail] &= (1 << (wl.d % 64)) - 1
    sb[tail + (1 if wl.d % 64 else 0):] = 0
    zb[tail + (1 if wl.d % 64 else 0):] = 0
    rs = np.random.default_rng(3)
    ranges = sample_ranges(wl, [0, 1], rs, width=8192, n_random=2)
    tb = th_dt == "bf16"
    for t in (1, 2):                                       # t = 2 averages tensor b
        g = gen.device_g(wl, t)
        pre = [(j0, j1, to_host(theta[j0:j1]).copy(), np.ascontiguousarray(to_host(m[:, j0:j1])),
                np.ascontiguousarray(to_host(g[:, j0:j1]))) for j0, j1 in ranges]
        lc.apply(theta, m, g, t, sb, zb)
        torch.cuda.synchronize()
        for j0, j1, th, mc, gc in pre:
            T = 0 if j1 <= wl.offsets[1] else 1
            sl = wl.with_(name="slice", tensors=[("b" if T else "a", j1 - j0)])
            lco.apply(sl, th, mc, gc, t, to_host(sb[j0 // 64:(j1 + 63) // 64]).view(np.uint64),
                      to_host(zb[j0 // 64:(j1 + 63) // 64]).view(np.uint64))
            check_float_state(f"theta[{j0}:{j1}] t={t}", to_host(theta[j0:j1]), th, bf16=tb)
            check_float_state(f"m[:, {j0}:{j1}] t={t}", to_host(m[:, j0:j1]), mc)
        _say("apply", dtypes, "t", t, "ok")
        del g
    lc.close()
    del theta, m, sb, zb
    torch.cuda.empty_cache()
