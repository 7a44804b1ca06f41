"""GPU parity: the gfx950 library against the CPU oracle on the same seeded
inputs, through the C ABI.  Sizes span several 4096-element blocks, more
than 64 blocks per tensor (several partials per finalize lane), ragged tail
quads, tensor boundaries, odd and even W, and the degenerate cases (exact
zeros, ties, a tensor whose mean |c| is 0, W = 1, W = 255)."""
import numpy as np
import pytest

from oracle import lco
from synth import workloads as wls
from tests.conftest import golden
from tests.harness import gpu_step_fn, gpu_step_vs_oracle, lioncub_for, to_dev, to_host

pytestmark = pytest.mark.gpu


def small(wl, cap, ntens=None):
    return wls.shrink(wl, cap, ntens)


WORKLOADS = {
    "flat-1M-w4-vote": wls.FLAT_1M_W4_VOTE,
    "gpt2-124M-w8-vote(small)": small(wls.GPT2_124M_W8_VOTE, 3 * 4096 + 640, 40),
    "flat-350M-w16-l1q4(small)": wls.FLAT_350M_W16_L1Q4.with_(
        tensors=[("flat", 70 * 4096 + 896)]),
    "gpt-760M-w8-vote-bf16-sync(small)": small(wls.GPT_760M_W8_VOTE_SYNC, 2 * 4096 + 192, 30),
    "gpt-1.3B-w8-l1q8-bf16g(small)": small(wls.GPT_1B3_W8_L1Q8, 2 * 4096 + 320, 30),
}


@pytest.mark.parametrize("debug", [True, False], ids=["debug", "production"])
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name, debug):
    wl = WORKLOADS[name]
    steps = 4 if wl.d < 4_000_000 else 2
    res = gpu_step_vs_oracle(wl, steps=steps, debug=debug)
    print(name, res, flush=True)


EDGE = {
    "ragged-d-W5-vote": wls.flat("e1", 2 * 4096 + 4099, W=5),
    "ragged-d-W5-l1": wls.flat("e2", 2 * 4096 + 4099, W=5, agg="l1", qbits=3),
    "W1-vote": wls.flat("e3", 5000, W=1),
    "W1-l1": wls.flat("e4", 5000, W=1, agg="l1", qbits=2),
    "W255-vote": wls.flat("e5", 1000, W=255),
    "W255-l1q8": wls.flat("e6", 1000, W=255, agg="l1", qbits=8),
    "W16-tiezero": wls.flat("e7", 9000, W=16, tie="zero"),
    "W6-tiezero-bf16": wls.flat("e8", 9000, W=6, tie="zero", theta_dtype="bf16",
                                grad_dtype="bf16"),
    "sync-every-2-vote": wls.Workload(name="e9", tensors=[("wte", 4096 + 64), ("h", 128),
                                                          ("wpe", 64)], W=4,
                                      sync_names=("wte", "wpe"), sync_every=2),
    "sync-every-2-l1": wls.Workload(name="e10", tensors=[("wte", 4096 + 64), ("h", 128),
                                                         ("wpe", 64)], W=3, agg="l1", qbits=4,
                                    sync_names=("wte", "wpe"), sync_every=2),
    "tiny-tensors": wls.Workload(name="e11", tensors=[("a", 64), ("b", 4096), ("c", 4160),
                                                      ("d", 64), ("e", 8192)], W=8, agg="l1",
                                 qbits=4),
    "row-padding": wls.flat("e12", 5000, W=8, ld_pad=128),
    "row-padding-l1": wls.flat("e13", 5000, W=16, agg="l1", qbits=4, ld_pad=192),
    "W16-bf16-both-l1": wls.flat("e14", 3 * 4096, W=16, agg="l1", qbits=4,
                                 theta_dtype="bf16", grad_dtype="bf16"),
    "W4-l1-generic-bf16g": wls.flat("e15", 3 * 4096 + 4, W=4, agg="l1", qbits=5,
                                    grad_dtype="bf16"),
    "W8-vote-f32-bf16theta": wls.flat("e16", 3 * 4096 + 8, W=8, theta_dtype="bf16"),
    # 255 momenta summed in fp32 in worker order for the synced tensor, every step
    "W255-l1q8-sync": wls.Workload(name="e17", tensors=[("wte", 640), ("h", 384)], W=255,
                                   agg="l1", qbits=8, sync_names=("wte",), sync_every=1),
    "W255-vote-bf16-sync": wls.Workload(name="e18", tensors=[("h", 4096 + 64), ("wpe", 128)],
                                        W=255, theta_dtype="bf16", grad_dtype="bf16",
                                        sync_names=("wpe",), sync_every=1),
    # padded rows with bf16 data and several tensors
    "row-padding-bf16-l1-tensors": wls.Workload(name="e19", tensors=[("a", 4096 + 192), ("b", 320)],
                                                W=6, agg="l1", qbits=6, theta_dtype="bf16",
                                                grad_dtype="bf16", ld_pad=256),
    "row-padding-bf16g-avg-sync": wls.Workload(name="e20", tensors=[("wte", 192), ("h", 4096 + 5)],
                                               W=5, agg="avg", grad_dtype="bf16", ld_pad=64,
                                               sync_names=("wte",), sync_every=3),
    # long tensor lists: 2,000 tensors of 64 to 4160 elements (tables built
    # in 63 launches of 32 entries; block and group owners found by search)
    "2000-tensors-vote": wls.Workload(name="e21", tensors=[(f"t{k}", 64 * (1 + k % 5) + (4096 if k % 97 == 0 else 0))
                                                           for k in range(2000)],
                                      W=3, sync_names=("t7", "t1999"), sync_every=2),
    "2000-tensors-l1": wls.Workload(name="e22", tensors=[(f"t{k}", 64 * (1 + k % 7) + (4096 if k % 89 == 0 else 0))
                                                         for k in range(2000)],
                                    W=4, agg="l1", qbits=5),
}


@pytest.mark.parametrize("debug", [True, False], ids=["debug", "production"])
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_parity(name, debug):
    wl = EDGE[name]
    res = gpu_step_vs_oracle(wl, steps=4, debug=debug)
    print(name, res, flush=True)


@pytest.mark.parametrize("t0", [2**62 - 1, 2**63 - 4], ids=["t=2^62-1", "t=2^63-4"])
def test_max_norm_counter_wraps(t0):
    """Step indices near 2^62 and 2^63: the max-norm draws' counter
    (t*W + i)*d + 2*floor(j/2) wraps modulo 2^64 on both sides (the
    wrap-around itself is pinned on the oracle by tuples landing on the
    generator's published outputs); the vote path's parity at the same t."""
    for wl in (wls.flat("wrap-linf", 3 * 4096 + 100, W=5, agg="linf", qbits=4),
               wls.Workload(name="wrap-linf-tensors", tensors=[("a", 4096 + 64), ("b", 704)], W=3,
                            agg="linf", qbits=7, grad_dtype="bf16"),
               wls.flat("wrap-vote", 4096 + 36, W=4, tie="zero")):
        res = gpu_step_vs_oracle(wl, steps=2, t0=t0)
        print(wl.name, t0, res, flush=True)


def test_vote_tie_rate_on_gpu():
    """Majority ties at W=4 occur for over 30% of parameters (the pages'
    observation; C(4,2)/16 = 0.375 for symmetric iid c)."""
    gd = golden("tie_rate.json")
    res = gpu_step_vs_oracle(wls.FLAT_1M_W4_VOTE, steps=1, zeros=False)
    rate = res["ties"] / wls.FLAT_1M_W4_VOTE.d
    assert abs(rate - gd["closed_form"]["4"]) < 0.005 and rate > gd["W4_min_rate"]


# ------------------------------------------------ standalone entry points --

def _ctx(W, d, ld=None, **kw):
    wl = wls.flat("api", d, W=W, **kw)
    if ld is not None:
        wl = wl.with_(ld_pad=ld - wl.ld)
    return wl, lioncub_for(wl)


@pytest.mark.parametrize("t,tie", [(1, "parity"), (2, "parity"), (1, "zero"), (2, "zero")])
def test_pack_vote_handworked(t, tie):
    """tests/golden/pack_vote_w4_d8.json through the library: bytes, counts
    and signs equal both the hand-worked values and the oracle."""
    import torch
    gd = golden("pack_vote_w4_d8.json")
    wl, lc = _ctx(4, 8, tie=tie)
    x = np.zeros((4, 64), np.float32)
    x[:, :8] = np.array(gd["x"], np.float32)
    bits = torch.full((4, 1), -1, dtype=torch.int64, device="cuda")
    lc.pack(to_dev(x), t, bits)
    counts = torch.zeros(8, dtype=torch.uint8, device="cuda")
    sign = torch.zeros(8, dtype=torch.int8, device="cuda")
    lc.vote(bits, t, counts, sign)
    torch.cuda.synchronize()
    want_bits = lco.pack(x, 8, t)
    assert np.array_equal(to_host(bits).view(np.uint64), want_bits)
    wc, ws = lco.vote(want_bits, 4, 8, t, lco.TIE_ZERO if tie == "zero" else lco.TIE_PARITY)
    assert np.array_equal(to_host(counts), wc)
    assert np.array_equal(to_host(sign), ws)
    want = gd["steps"][str(t)]
    assert [int(w) for w in to_host(bits)[:, 0]] == want["bytes"]
    assert to_host(counts).tolist() == want["counts"]
    assert to_host(sign).tolist() == want["sign_zero" if tie == "zero" else "sign_parity"]
    lc.close()


@pytest.mark.parametrize("d", [3 * 4096 + 1001, 3 * 16384 + 1001, 4 * 16384])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 17, 40, 255])
@pytest.mark.parametrize("t", [1, 2])
def test_pack_vote_random(W, t, d):
    """Ragged d, exact zeros, padded rows; bitwise against the oracle (whose
    pack and vote are pinned by brute force and NumPy's packbits).  The
    larger sizes span several full vote workgroups (256 words: the
    LDS-staged store path) and a partial last one."""
    import torch
    rs = np.random.default_rng(W * 10 + t)
    ld = (d + 63) // 64 * 64 + 128
    wl, lc = _ctx(W, d, ld=ld)
    x = rs.standard_normal((W, ld)).astype(np.float32)
    x[rs.random((W, ld)) < 0.05] = 0.0
    x[:, ::7] *= -0.0
    bits = torch.full((W, ld // 64), -1, dtype=torch.int64, device="cuda")
    lc.pack(to_dev(x), t, bits)
    counts = torch.zeros(d, dtype=torch.uint8, device="cuda")
    sign = torch.zeros(d, dtype=torch.int8, device="cuda")
    lc.vote(bits, t, counts, sign)
    only_sign = torch.zeros(d, dtype=torch.int8, device="cuda")
    lc.vote(bits, t, None, only_sign)
    only_counts = torch.zeros(d, dtype=torch.uint8, device="cuda")
    lc.vote(bits, t, only_counts, None)
    torch.cuda.synchronize()
    wb = lco.pack(x, d, t)
    assert np.array_equal(to_host(bits).view(np.uint64), wb)
    wc, ws = lco.vote(wb, W, d, t)
    assert np.array_equal(to_host(counts), wc)
    assert np.array_equal(to_host(sign), ws)
    assert np.array_equal(to_host(only_sign), ws)
    assert np.array_equal(to_host(only_counts), wc)
    lc.close()


def _quant_case(x, tensors, qbits):
    import torch
    W, ld = x.shape
    wl = wls.Workload(name="q", tensors=tensors, W=W, agg="l1", qbits=qbits)
    wl = wl.with_(ld_pad=ld - wl.ld)
    lc = lioncub_for(wl)
    codes = torch.full((W, ld), 99, dtype=torch.int8, device="cuda")
    m1 = torch.zeros((W, wl.n_tensors), dtype=torch.float64, device="cuda")
    lc.quant_l1(to_dev(x), codes, m1)
    torch.cuda.synchronize()
    wc, wm = lco.quant_l1(wl, x)
    gm = to_host(m1)
    assert np.array_equal(gm.view(np.uint64), wm.view(np.uint64)), (gm, wm)
    gc = to_host(codes)
    assert np.array_equal(gc[:, : wl.d], wc[:, : wl.d])
    assert np.all(gc[:, wl.d:] == 99)           # columns past d untouched
    lc.close()


def test_quant_l1_handworked():
    x = np.zeros((1, 64), np.float32)
    x[0, :8] = [0.5, -0.1, 0, 2, -3, 0.25, 0.05, -0.05]
    _quant_case(x, [("a", 8)], 4)
    x = np.zeros((1, 64), np.float32)
    x[0, :4] = [0.5, -0.5, 1.5, -1.5]
    _quant_case(x, [("a", 4)], 2)
    x = np.zeros((1, 64), np.float32)
    x[0, :5] = [0.5, 1.5, 2.5, -2.5, 8.0]
    _quant_case(x, [("a", 5)], 3)


def test_fp32_evaluation_order_handworked_gpu():
    """The library's theta and averaged-momentum arithmetic against values
    worked by hand where another evaluation order or a fused multiply-add
    would round differently (tests/golden/fp32_order.json), not against the
    oracle."""
    import torch

    from tests.test_oracle_pins import fp32_order_average_run, fp32_order_theta_run

    def step(wl, theta, m, g, want_m=False):
        lc = lioncub_for(wl)
        th = to_dev(theta if theta is not None else np.zeros(wl.d, np.float32))
        dm = to_dev(m)
        lc.step(th, dm, to_dev(g), 1)
        torch.cuda.synchronize()
        lc.close()
        return to_host(dm) if want_m else to_host(th)

    gd = golden("fp32_order.json")
    for case in gd["theta_cases"]:
        assert np.all(fp32_order_theta_run(step, case) == int(case["theta_next_hex"], 16)), \
            case["name"]
    want = np.array([int(h, 16) for h in gd["average_case"]["m_next_hex"]], np.uint32)
    assert np.all(fp32_order_average_run(step) == want[None, :])


@pytest.mark.parametrize("t", [1, 2])
def test_tie_rule_handworked_gpu(t):
    """Both tie rules on columns that tie by construction: applied sign,
    theta and the diagnostics' counts against values fixed by hand."""
    from tests.test_oracle_pins import tie_rule_run
    tie_rule_run(gpu_step_fn(), t)


def test_bf16_theta_decay_handworked_gpu():
    from tests.test_oracle_pins import bf16_decay_run
    bf16_decay_run(gpu_step_fn())


def test_bf16_theta_nan_narrows_to_quiet_nan_gpu():
    """bf16 parameters that are NaN (any sign and payload) stay NaN through
    the step and come back as the quiet NaN 0x7FC0; the finite ones equal
    the oracle's."""
    from synth.gen import to_bf16_bits
    wl = wls.flat("nan", 300, W=3, theta_dtype="bf16", grad_dtype="bf16")
    rs = np.random.default_rng(8)
    theta = to_bf16_bits(rs.normal(0, 0.02, 300).astype(np.float32))
    nans = np.array([0x7F81, 0xFF81, 0x7FC0, 0xFFC0, 0x7FFF, 0xFFFF, 0x7FA0], np.uint16)
    theta[::43] = nans[: len(theta[::43])]
    g = np.zeros((3, wl.ld), np.uint16)
    g[:, :300] = to_bf16_bits(rs.normal(0, 1e-3, (3, 300)).astype(np.float32))
    m = np.zeros((3, wl.ld), np.float32)
    got = gpu_step_fn()(wl, theta, m, g, 1)["theta"]
    want = theta.copy()
    lco.step(wl, want, m.copy(), g.copy(), 1)
    assert np.all(got[::43] == 0x7FC0)
    assert np.array_equal(got, want)


def test_identical_momenta_zero_spread_gpu():
    """64 identical workers: the largest inter-worker variance is exactly 0
    although its fp64 evaluation is negative for some columns."""
    from tests.test_oracle_pins import zero_spread_run
    zero_spread_run(gpu_step_fn())


def test_quant_l1_scale_precision_gpu():
    """Eq. (1) on a row whose first code sits 1.65e-8 below a rounding
    boundary, worked in exact arithmetic: the standalone quantiser and the
    fused step's codes (c = x with beta1 = 1/2, m = 0, g = 2x)."""
    import torch

    from tests.test_oracle_pins import scale_precision_run

    def standalone(x, n):
        wl = wls.flat("sp", x.size, W=1, agg="l1", qbits=n)
        xx = np.zeros((1, wl.ld), np.float32)
        xx[0, : x.size] = x
        lc = lioncub_for(wl)
        codes = torch.zeros((1, wl.ld), dtype=torch.int8, device="cuda")
        m1 = torch.zeros((1, 1), dtype=torch.float64, device="cuda")
        lc.quant_l1(to_dev(xx), codes, m1)
        torch.cuda.synchronize()
        lc.close()
        return to_host(codes)[0, : x.size], float(to_host(m1)[0, 0])

    def fused(x, n):
        wl = wls.flat("sp", x.size, W=1, agg="l1", qbits=n, beta1=0.5)
        g = np.zeros((1, wl.ld), np.float32)
        g[0, : x.size] = np.float32(2) * x
        out = gpu_step_fn()(wl, np.zeros(x.size, np.float32), np.zeros((1, wl.ld), np.float32),
                            g, 1)
        return out["codes"][0, : x.size], float(out["m1"][0, 0])

    scale_precision_run(standalone)
    scale_precision_run(fused)


def _m1_order_rows(cases, W):
    """The hand-worked summation-order cases as consecutive tensors; worker
    i holds the case vectors scaled by (-2)^i (exact at every tree level)."""
    wl = wls.Workload(name="m1order", tensors=[(c["name"], c["n"]) for c in cases], W=W,
                      agg="l1", qbits=4)
    x = np.zeros((W, wl.ld), np.float32)
    for T, c in enumerate(cases):
        a = wl.offsets[T]
        for k, e in c["place"]:
            for i in range(W):
                x[i, a + k] = np.float32((-2.0) ** i * 2.0**e)
    return wl, x


def _m1_worked(c):
    from fractions import Fraction
    return float(Fraction(float.fromhex(c["S"])) / c["n"])


@pytest.mark.parametrize("big", [False, True], ids=["tensors", "many-groups"])
def test_m1_order_handworked_gpu(big):
    """The library's mean |x| against sums worked by hand from the written
    summation order (tests/golden/m1_order.json), not against the oracle:
    quad pairing, rounds in order, wave halving, block nesting, the group
    fold, the final lanes over 34 and 65 groups of 256 blocks, the divisor.
    Through the standalone quantiser (m1 output) and through the fused
    step's norm pass (beta1 = 1/2, g = 0: c = m/2 exactly, so M1 halves)."""
    import torch
    cases = golden("m1_order.json")["cases"]
    if big:
        groups = [[c] for c in cases if c["n"] > (1 << 20)]
    else:
        small_cases = [c for c in cases if c["n"] <= (1 << 20)]
        groups = [sorted(small_cases, key=lambda c: c["n"] % 64 != 0)]
    for cs in groups:
        W = 1 if big else 2
        wl, x = _m1_order_rows(cs, W)
        want = np.array([[2.0**i * _m1_worked(c) for c in cs] for i in range(W)])
        lc = lioncub_for(wl)
        codes = torch.zeros((W, wl.ld), dtype=torch.int8, device="cuda")
        m1 = torch.zeros((W, wl.n_tensors), dtype=torch.float64, device="cuda")
        lc.quant_l1(to_dev(x), codes, m1)
        torch.cuda.synchronize()
        got = to_host(m1)
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), (got, want)
        lc.close()
        for gdt in ("f32", "bf16"):
            wl2 = wl.with_(beta1=0.5, grad_dtype=gdt)
            lc = lioncub_for(wl2)
            theta = torch.zeros(wl.d, dtype=torch.float32, device="cuda")
            d_m = to_dev(x)
            g = torch.zeros((W, wl.ld), dtype=torch.bfloat16 if gdt == "bf16" else torch.float32,
                            device="cuda")
            m1s = torch.zeros((W, wl.n_tensors), dtype=torch.float64, device="cuda")
            lc.step(theta, d_m, g, 1, {"m1": m1s})
            torch.cuda.synchronize()
            got = to_host(m1s)
            assert np.array_equal(got.view(np.uint64), (want * 0.5).view(np.uint64)), (got, want)
            lc.close()
        del x
        print("m1 order", [c["name"] for c in cs], "ok", flush=True)


@pytest.mark.parametrize("qbits", [2, 4, 8])
def test_quant_l1_adversarial_magnitudes(qbits):
    """Magnitudes over 1e-30..1e30 make the fp64 sum order-sensitive: the
    mean must still agree to the bit (the fixed summation tree), and so must
    every code.  Also a tensor of zeros (mean 0 -> codes 0), subnormals, and
    more than 64 blocks in one tensor."""
    rs = np.random.default_rng(qbits)
    tensors = [("a", 70 * 4096 + 832), ("z", 128), ("s", 4096 + 64)]
    d = sum(n for _, n in tensors)
    W = 3
    ld = (d + 63) // 64 * 64
    x = (10.0 ** rs.uniform(-30, 30, (W, ld)) * np.where(rs.random((W, ld)) < 0.5, -1, 1))
    x = x.astype(np.float32)
    a, b = tensors[0][1], tensors[0][1] + 128
    x[:, a:b] = 0.0
    x[1, b:d] = (rs.integers(1, 100, d - b) * 1e-45).astype(np.float32)   # subnormals
    _quant_case(x, tensors, qbits)


def test_quant_l1_student_t():
    rs = np.random.default_rng(5)
    tensors = [("a", 9 * 4096 + 320), ("b", 64)]
    d = sum(n for _, n in tensors)
    x = (rs.standard_t(2.5, (16, d)) * 1e-3).astype(np.float32)
    _quant_case(x, tensors, 4)


# ----------------------------------------------------- state properties --

def test_deterministic_and_checkpoint_resume():
    """Same inputs twice -> identical bits; 6 steps straight == 3 steps, a
    host round trip of (theta, m, t), then 3 more."""
    import torch
    from synth import gen
    wl = wls.flat("ck", 5 * 4096 + 96, W=8, agg="l1", qbits=4)
    theta0, m0 = gen.host_theta(wl), gen.host_m(wl)
    gs = [to_dev(gen.host_g(wl, t)) for t in range(1, 7)]

    def run(ts, th, m):
        lc = lioncub_for(wl)
        for t in ts:
            lc.step(th, m, gs[t - 1], t)
        torch.cuda.synchronize()
        lc.close()

    thA, mA = to_dev(theta0), to_dev(m0)
    run(range(1, 7), thA, mA)
    thB, mB = to_dev(theta0), to_dev(m0)
    run(range(1, 7), thB, mB)
    assert torch.equal(thA, thB) and torch.equal(mA, mB)
    thC, mC = to_dev(theta0), to_dev(m0)
    run(range(1, 4), thC, mC)
    th_h, m_h = to_host(thC).copy(), to_host(mC).copy()
    thD, mD = to_dev(th_h), to_dev(m_h)
    run(range(4, 7), thD, mD)
    assert torch.equal(thA, thD) and torch.equal(mA, mD)


def test_bad_arguments_on_device():
    import torch
    from communication_compressed_distributed_amd import LionCubError, _abi
    wl, lc = _ctx(4, 4096)
    th = torch.zeros(4096, device="cuda")
    m = torch.zeros((4, 4096), device="cuda")
    with pytest.raises(LionCubError):
        lc.step(th, m, m, 0)                              # t must be >= 1
    with pytest.raises(LionCubError):                      # misaligned theta, raw ABI
        _abi.lioncub_step(lc.ctx, th[1:], m, m, 1)
    with pytest.raises(ValueError):                       # too short: caught on the host
        lc.step(th[1:], m, m, 1)
    with pytest.raises(ValueError):
        lc.step(th, m[:, :2048], m, 1)                    # strided view of m
    with pytest.raises(ValueError):
        lc.step(th, m, m.to(torch.bfloat16), 1)           # g dtype differs from the config
    with pytest.raises(ValueError):
        lc.step(th.cpu(), m, m, 1)                        # host tensor
    with pytest.raises(LionCubError):
        lc.step(th, m, m, 1, {"codes": torch.zeros((4, 4096), dtype=torch.int8,
                                                   device="cuda")})  # L1 output on vote path
    with pytest.raises(LionCubError):
        lc.vote(torch.zeros((4, 64), dtype=torch.int64, device="cuda"), 1)  # no output
    with pytest.raises(LionCubError):
        lc.quant_l1(m, torch.zeros((4, 4096), dtype=torch.int8, device="cuda"))  # no qbits
    lc.close()


# -------------------- D-Lion averaging, receive side and wire formats ----

AVG = {
    "avg-W4": wls.flat("a1", 3 * 4096 + 300, W=4, agg="avg"),
    "avg-W3-bf16": wls.flat("a2", 2 * 4096 + 4099, W=3, agg="avg", theta_dtype="bf16",
                            grad_dtype="bf16"),
    "avg-W16-sync": wls.Workload(name="a3", tensors=[("wte", 4096 + 64), ("h", 8192)], W=16,
                                 agg="avg", sync_names=("wte",), sync_every=2),
    "avg-W8-gpt": small(wls.GPT2_124M_W8_VOTE.with_(agg="avg"), 4096 + 640, 20),
    "avg-W255-sync": wls.Workload(name="a5", tensors=[("wte", 640), ("h", 4096 + 64)], W=255,
                                  agg="avg", sync_names=("wte",), sync_every=1),
}


@pytest.mark.parametrize("debug", [True, False], ids=["debug", "production"])
@pytest.mark.parametrize("name", list(AVG))
def test_avg_parity(name, debug):
    res = gpu_step_vs_oracle(AVG[name], steps=3, debug=debug)
    print(name, res, flush=True)


@pytest.mark.parametrize("W", [1, 3, 4, 8, 16, 255])
@pytest.mark.parametrize("tie", ["parity", "zero"])
def test_vote_bits_parity(W, tie):
    import torch
    rs = np.random.default_rng(W)
    d = 2 * 4096 + 777
    ld = (d + 63) // 64 * 64 + 64
    wl, lc = _ctx(W, d, ld=ld, tie=tie)
    tm = lco.TIE_ZERO if tie == "zero" else lco.TIE_PARITY
    for t in (1, 2):
        x = rs.standard_normal((W, ld)).astype(np.float32)
        x[rs.random((W, ld)) < 0.05] = 0.0
        bits = lco.pack(x, d, t)
        sb = torch.full((ld // 64,), -1, dtype=torch.int64, device="cuda")
        zb = torch.full((ld // 64,), -1, dtype=torch.int64, device="cuda")
        lc.vote_bits(to_dev(bits.view(np.int64)), t, sb, zb)
        sb1 = torch.full((ld // 64,), -1, dtype=torch.int64, device="cuda")
        lc.vote_bits(to_dev(bits.view(np.int64)), t, sb1)
        torch.cuda.synchronize()
        wsb, wzb = lco.vote_bits(bits, W, d, t, tm)
        assert np.array_equal(to_host(sb).view(np.uint64), wsb)
        assert np.array_equal(to_host(zb).view(np.uint64), wzb)
        assert np.array_equal(to_host(sb1).view(np.uint64), wsb)
    lc.close()


APPLY = {
    "apply-W4": wls.flat("p1", 3 * 4096 + 300, W=4),
    "apply-W16-l1cfg": wls.flat("p2", 2 * 4096 + 4099, W=16, agg="l1", qbits=4),
    "apply-W5-bf16-sync": wls.Workload(name="p3", tensors=[("wte", 4096 + 64), ("h", 4160)], W=5,
                                       theta_dtype="bf16", grad_dtype="bf16",
                                       sync_names=("wte",), sync_every=1),
    "apply-W8-gpt": small(wls.GPT_760M_W8_VOTE_SYNC, 4096 + 640, 20),
}


@pytest.mark.parametrize("zero", [True, False])
@pytest.mark.parametrize("name", list(APPLY))
def test_apply_parity(name, zero):
    import torch
    from synth import gen
    wl = APPLY[name]
    rs = np.random.default_rng(3)
    tb, gb = wl.theta_dtype == "bf16", wl.grad_dtype == "bf16"
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    lc = lioncub_for(wl)
    d_theta, d_m = to_dev(theta, tb), to_dev(m)
    for t in (1, 2, 3):
        g = gen.host_g(wl, t)
        s = rs.integers(-1 if zero else 0, 2, wl.ld)
        if not zero:
            s = np.where(s == 0, -1, 1)
        s[wl.d:] = 0
        sb = np.packbits(s > 0, bitorder="little").view("<u8").copy()
        zb = np.packbits(s == 0, bitorder="little").view("<u8").copy() if zero else None
        lc.apply(d_theta, d_m, to_dev(g, gb), t, to_dev(sb.view(np.int64)),
                 None if zb is None else to_dev(zb.view(np.int64)))
        torch.cuda.synchronize()
        lco.apply(wl, theta, m, g, t, sb, zb)
        from tests.harness import check_float_state
        check_float_state(f"theta t={t}", to_host(d_theta), theta, bf16=tb)
        check_float_state(f"m t={t}", to_host(d_m)[:, :wl.d], m[:, :wl.d])
    lc.close()


@pytest.mark.parametrize("W", [4, 8, 16])
def test_one_bit_path_composes_into_the_step(W):
    """The worker-sharded 1-bit flow on one GPU: pack(c) -> vote_bits ->
    apply gives exactly what the fused step gives (theta and m bit for bit)."""
    import torch
    from synth import gen
    wl = wls.flat("c1b", 3 * 4096 + 128, W=W)
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    g = gen.host_g(wl, 1)
    c = np.zeros((W, wl.ld), np.float32)
    for i in range(W):
        c[i, : wl.d] = lco.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    lc = lioncub_for(wl)
    thA, mA, dg = to_dev(theta), to_dev(m), to_dev(g)
    lc.step(thA, mA, dg, 1)
    thB, mB = to_dev(theta), to_dev(m)
    bits = torch.empty((W, wl.ld // 64), dtype=torch.int64, device="cuda")
    sb = torch.empty((wl.ld // 64,), dtype=torch.int64, device="cuda")
    lc.pack(to_dev(c), 1, bits)
    lc.vote_bits(bits, 1, sb)
    lc.apply(thB, mB, dg, 1, sb)
    torch.cuda.synchronize()
    assert torch.equal(thA, thB) and torch.equal(mA, mB)
    lc.close()


@pytest.mark.parametrize("d", [4096 + 1000 + 7, 3 * 8192 + 1000 + 7, 4 * 8192])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("W", [1, 3, 16])
def test_wire_pack_and_unpack_sum(n, W, d):
    """Sizes from one partial workgroup to several full unpack workgroups
    (8192 elements each) and a partial last one; row padding past d."""
    import torch
    qmax = 2 ** (n - 1) - 1
    rs = np.random.default_rng(10 * n + W)
    ld = (d + 63) // 64 * 64 + 64
    wl, lc = _ctx(W, d, ld=ld, agg="l1", qbits=n)
    codes = rs.integers(-qmax, qmax + 1, (W, ld)).astype(np.int8)   # junk past d too
    wire = torch.full((W, (ld // 32) * n), -1, dtype=torch.int32, device="cuda")
    lc.pack_codes(to_dev(codes), wire)
    sums = torch.zeros(d, dtype=torch.int32, device="cuda")
    sign = torch.zeros(d, dtype=torch.int8, device="cuda")
    lc.unpack_sum(wire, sums, sign)
    only_sign = torch.zeros(d, dtype=torch.int8, device="cuda")
    lc.unpack_sum(wire, None, only_sign)
    only_sums = torch.zeros(d, dtype=torch.int32, device="cuda")
    lc.unpack_sum(wire, only_sums, None)
    torch.cuda.synchronize()
    ww = lco.pack_codes(codes, d, n)
    assert np.array_equal(to_host(wire).view(np.uint32), ww)
    ws, wsg = lco.unpack_sum(ww, W, d, ld, n)
    assert np.array_equal(to_host(sums), ws)
    assert np.array_equal(to_host(sign), wsg)
    assert np.array_equal(to_host(only_sign), wsg)
    assert np.array_equal(to_host(only_sums), ws)
    lc.close()


@pytest.mark.parametrize("d", [4096 + 1000 + 7, 3 * 8192 + 1000 + 7, 4 * 8192])
@pytest.mark.parametrize("n", [2, 3, 4, 8])
@pytest.mark.parametrize("W", [1, 3, 16])
def test_unpack_sum_bits(n, W, d):
    """Sign and zero planes of the p-bit sums against the oracle, with row
    padding: words wholly past d are written as 0 (the planes start as
    junk); the zero plane is optional."""
    import torch
    qmax = 2 ** (n - 1) - 1
    rs = np.random.default_rng(100 + 10 * n + W)
    ld = (d + 63) // 64 * 64 + 128
    wl, lc = _ctx(W, d, ld=ld, agg="l1", qbits=n)
    codes = rs.integers(-qmax, qmax + 1, (W, ld)).astype(np.int8)
    codes[:, 64:192] = 0                                   # exact zero sums
    wire = torch.empty((W, (ld // 32) * n), dtype=torch.int32, device="cuda")
    lc.pack_codes(to_dev(codes), wire)
    sb = torch.full((ld // 64,), -1, dtype=torch.int64, device="cuda")
    zb = torch.full((ld // 64,), -1, dtype=torch.int64, device="cuda")
    lc.unpack_sum_bits(wire, sb, zb)
    sb_only = torch.full((ld // 64,), -1, dtype=torch.int64, device="cuda")
    lc.unpack_sum_bits(wire, sb_only)
    torch.cuda.synchronize()
    ws, wz = lco.unpack_sum_bits(to_host(wire).view(np.uint32), W, d, ld, n)
    assert np.array_equal(to_host(sb).view(np.uint64), ws)
    assert np.array_equal(to_host(zb).view(np.uint64), wz)
    assert np.array_equal(to_host(sb_only).view(np.uint64), ws)
    lc.close()


@pytest.mark.parametrize("n", [3, 4, 8])
def test_p_bit_exchange_composes_into_the_step(n):
    """The worker-sharded p-bit flow on one GPU: quant_l1(c) -> pack_codes ->
    unpack_sum_bits -> apply gives theta and m bit for bit equal to the
    fused L1 step, on two tensors with a ragged end and bf16 gradients."""
    import torch
    from synth import gen
    wl = wls.Workload(name="pbx", tensors=[("a", 2 * 4096 + 192), ("b", 4096)], W=8, agg="l1",
                      qbits=n, grad_dtype="bf16")
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    g = gen.host_g(wl, 1)
    c = np.zeros((wl.W, wl.ld), np.float32)
    for i in range(wl.W):
        c[i, : wl.d] = lco.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    lc = lioncub_for(wl)
    dg = to_dev(g, bf16=True)
    thA, mA = to_dev(theta), to_dev(m)
    lc.step(thA, mA, dg, 3)
    codes = torch.zeros((wl.W, wl.ld), dtype=torch.int8, device="cuda")
    lc.quant_l1(to_dev(c), codes)
    wire = torch.empty((wl.W, (wl.ld // 32) * n), dtype=torch.int32, device="cuda")
    lc.pack_codes(codes, wire)
    sb = torch.empty((wl.ld // 64,), dtype=torch.int64, device="cuda")
    zb = torch.empty((wl.ld // 64,), dtype=torch.int64, device="cuda")
    lc.unpack_sum_bits(wire, sb, zb)
    thB, mB = to_dev(theta), to_dev(m)
    lc.apply(thB, mB, dg, 3, sb, zb)
    torch.cuda.synchronize()
    assert int(to_host(zb).view(np.uint64).astype(bool).sum()) > 0   # zeros were exercised
    assert torch.equal(thA, thB) and torch.equal(mA, mB)
    lc.close()


def test_p_bit_path_composes_into_the_step():
    """quant_l1(c) -> pack_codes -> unpack_sum reproduces the fused L1 step's
    integer sums and signs (debug outputs) bit for bit."""
    import torch
    from synth import gen
    wl = wls.Workload(name="pb", tensors=[("a", 2 * 4096 + 192), ("b", 4096)], W=8, agg="l1",
                      qbits=4)
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    g = gen.host_g(wl, 1)
    c = np.zeros((wl.W, wl.ld), np.float32)
    for i in range(wl.W):
        c[i, : wl.d] = lco.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    lc = lioncub_for(wl)
    dbg = {"sums": torch.zeros(wl.d, dtype=torch.int32, device="cuda"),
           "sign": torch.zeros(wl.d, dtype=torch.int8, device="cuda")}
    lc.step(to_dev(theta), to_dev(m), to_dev(g), 1, dbg)
    codes = torch.zeros((wl.W, wl.ld), dtype=torch.int8, device="cuda")
    lc.quant_l1(to_dev(c), codes)
    wire = torch.empty((wl.W, (wl.ld // 32) * wl.qbits), dtype=torch.int32, device="cuda")
    lc.pack_codes(codes, wire)
    sums = torch.zeros(wl.d, dtype=torch.int32, device="cuda")
    sign = torch.zeros(wl.d, dtype=torch.int8, device="cuda")
    lc.unpack_sum(wire, sums, sign)
    torch.cuda.synchronize()
    assert torch.equal(sums, dbg["sums"]) and torch.equal(sign, dbg["sign"])
    lc.close()


# ------------------------------- max-norm stochastic baseline (Q-inf) -----
# Parity here is bit-exact against the oracle's reading of the quantiser
# (the pages name it but do not print its formula).

LINF = {
    "linf-flat-W16-q4": wls.FLAT_350M_W16_L1Q4.with_(tensors=[("flat", 70 * 4096 + 896)],
                                                     agg="linf"),
    "linf-gpt-W8-q8-bf16g(small)": small(wls.GPT_1B3_W8_L1Q8, 2 * 4096 + 320, 30).with_(
        agg="linf"),
    "linf-ragged-W5-q3": wls.flat("i1", 2 * 4096 + 4099, W=5, agg="linf", qbits=3),
    "linf-W1-q2": wls.flat("i2", 5000, W=1, agg="linf", qbits=2),
    "linf-W255-q8": wls.flat("i3", 1000, W=255, agg="linf", qbits=8),
    "linf-sync-every-2-bf16": wls.Workload(name="i4", tensors=[("wte", 4096 + 64), ("h", 128),
                                                               ("wpe", 64)], W=3, agg="linf",
                                           qbits=4, sync_names=("wte", "wpe"), sync_every=2,
                                           theta_dtype="bf16", grad_dtype="bf16"),
    "linf-tiny-tensors-W8": wls.Workload(name="i5", tensors=[("a", 64), ("b", 4096),
                                                             ("c", 4160), ("d", 64)], W=8,
                                         agg="linf", qbits=4, sr_seed=2**64 - 1),
    "linf-row-padding-W16": wls.flat("i6", 5000, W=16, agg="linf", qbits=4, ld_pad=192),
    "linf-W4-generic-bf16g": wls.flat("i7", 3 * 4096 + 4, W=4, agg="linf", qbits=5,
                                      grad_dtype="bf16"),
}


@pytest.mark.parametrize("debug", [True, False], ids=["debug", "production"])
@pytest.mark.parametrize("name", list(LINF))
def test_linf_parity(name, debug):
    wl = LINF[name]
    res = gpu_step_vs_oracle(wl, steps=3, debug=debug)
    print(name, res, flush=True)


def test_linf_counter_wraps_like_the_oracle():
    """Step indices near 2^62: (t*W + i)*d wraps mod 2^64 on both sides."""
    wl = wls.flat("iw", 2 * 4096 + 64, W=3, agg="linf", qbits=4)
    res = gpu_step_vs_oracle(wl, steps=2, t0=2**62 + 5, debug=True)
    print(res, flush=True)


def _quant_linf_case(x, tensors, qbits, t, seed=0x5EED):
    import torch
    W, ld = x.shape
    wl = wls.Workload(name="qi", tensors=tensors, W=W, agg="linf", qbits=qbits, sr_seed=seed)
    wl = wl.with_(ld_pad=ld - wl.ld)
    lc = lioncub_for(wl)
    codes = torch.full((W, ld), 99, dtype=torch.int8, device="cuda")
    mv = torch.zeros((W, wl.n_tensors), dtype=torch.float64, device="cuda")
    lc.quant_linf(to_dev(x), t, codes, mv)
    torch.cuda.synchronize()
    wc, wm = lco.quant_linf(wl, x, t)
    gm = to_host(mv)
    assert np.array_equal(gm.view(np.uint64), wm.view(np.uint64)), (gm, wm)
    gc = to_host(codes)
    assert np.array_equal(gc[:, : wl.d], wc[:, : wl.d])
    assert np.all(gc[:, wl.d:] == 99)           # columns past d untouched
    lc.close()
    return gc[:, : wl.d]


@pytest.mark.parametrize("qbits", [2, 4, 8])
@pytest.mark.parametrize("t", [1, 2, 2**62 + 1])
def test_quant_linf_student_t(qbits, t):
    rs = np.random.default_rng(qbits)
    tensors = [("a", 9 * 4096 + 320), ("z", 128), ("b", 64)]
    d = sum(n for _, n in tensors)
    x = (rs.standard_t(2.5, (16, d)) * 1e-3).astype(np.float32)
    x[:, 9 * 4096 + 320: 9 * 4096 + 448] = 0.0               # a tensor of zeros
    codes = _quant_linf_case(x, tensors, qbits, t)
    if qbits <= 4:                                            # most codes 0 on heavy tails
        assert np.mean(codes[:, : 9 * 4096 + 320] == 0) > 0.5


def test_quant_linf_adversarial_magnitudes():
    """Magnitudes over 1e-30..1e30, subnormals, more than 64 blocks."""
    rs = np.random.default_rng(17)
    tensors = [("a", 70 * 4096 + 832), ("s", 4096 + 64)]
    d = sum(n for _, n in tensors)
    W, ld = 3, (d + 63) // 64 * 64
    x = (10.0 ** rs.uniform(-30, 30, (W, ld)) * np.where(rs.random((W, ld)) < 0.5, -1, 1))
    x = x.astype(np.float32)
    a = tensors[0][1]
    x[1, a:d] = (rs.integers(1, 100, d - a) * 1e-45).astype(np.float32)
    _quant_linf_case(x, tensors, 4, 3, seed=12345)


def test_linf_step_codes_are_quant_linf_of_c():
    """The fused step's codes at step t are quant_linf(c, t) on the device."""
    import torch
    from synth import gen
    wl = wls.Workload(name="ic", tensors=[("a", 2 * 4096 + 192), ("b", 4096)], W=8,
                      agg="linf", qbits=4, grad_dtype="bf16")
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    g = gen.host_g(wl, 7)
    c = np.zeros((wl.W, wl.ld), np.float32)
    for i in range(wl.W):
        c[i, : wl.d] = lco.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    lc = lioncub_for(wl)
    dbg = {"codes": torch.zeros((wl.W, wl.ld), dtype=torch.int8, device="cuda"),
           "m1": torch.zeros((wl.W, wl.n_tensors), dtype=torch.float64, device="cuda")}
    lc.step(to_dev(theta), to_dev(m), to_dev(g, True), 7, dbg)
    codes = torch.zeros((wl.W, wl.ld), dtype=torch.int8, device="cuda")
    mv = torch.zeros((wl.W, wl.n_tensors), dtype=torch.float64, device="cuda")
    lc.quant_linf(to_dev(c), 7, codes, mv)
    torch.cuda.synchronize()
    assert torch.equal(codes[:, : wl.d], dbg["codes"][:, : wl.d])
    assert torch.equal(mv, dbg["m1"])
    lc.close()


# ------------------------------------------------- more edges, all paths --

@pytest.mark.parametrize("agg", ["l1", "linf"])
@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7, 8])
def test_every_code_width_on_the_step(agg, n):
    wl = wls.flat(f"n{n}", 2 * 4096 + 33, W=5, agg=agg, qbits=n, grad_dtype="bf16")
    gpu_step_vs_oracle(wl, steps=2, debug=True)


@pytest.mark.parametrize("agg", ["vote", "avg", "l1", "linf"])
@pytest.mark.parametrize("d,W", [(1, 3), (1, 2), (63, 7), (64, 1), (65, 16)])
def test_tiny_vectors(agg, d, W):
    wl = wls.flat("tiny", d, W=W, agg=agg, qbits=0 if agg in ("vote", "avg") else 4)
    gpu_step_vs_oracle(wl, steps=3, debug=True)
    gpu_step_vs_oracle(wl, steps=1, debug=False, seed_shift=1)


@pytest.mark.parametrize("agg", ["vote", "l1", "linf"])
def test_sync_every_ten_over_twelve_steps(agg):
    """The pages' interval: momentum of the embedding tensors averaged every
    10 steps.  Twelve consecutive steps from t = 1, compared after each, so
    step 10 averages and steps 1-9, 11, 12 do not."""
    wl = wls.Workload(name="s10", tensors=[("wte", 2 * 4096 + 64), ("h", 4096 + 128),
                                           ("wpe", 128)], W=4, agg=agg,
                      qbits=0 if agg == "vote" else 4, sync_names=("wte", "wpe"), sync_every=10,
                      theta_dtype="bf16", grad_dtype="bf16")
    gpu_step_vs_oracle(wl, steps=12, t0=1, debug=True)
