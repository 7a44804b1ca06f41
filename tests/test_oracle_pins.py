"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what it pins the oracle to: a closed form of the Lion
recurrence, a hand-worked example from the definitions on the Lion Cub page
(pith.science review, "What carries the argument" and Eq. (1)), brute force
over every sign pattern, exact rational arithmetic, a library routine (NumPy's
bit packing, Python's correctly rounded math.fsum, torch's bf16 conversion),
an invariant, or a statistical property the pages state (the majority-vote tie
rate).  No expected value here is produced by the GPU library.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from synth import workloads as wls
from synth.gen import bf16_bits_to_f32
from tests.conftest import golden


def one_tensor(d, W, **kw):
    return wls.flat("pin", d, W=W, **kw)


# ------------------------------------------------------------------ bf16 --

def test_bf16_rounding_matches_torch(oracle):
    """fp32 -> bf16 round-to-nearest-even equals torch's conversion."""
    import torch
    rs = np.random.default_rng(1)
    bits = rs.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]            # finite only
    ties = (rs.integers(0, 2**16, 2000, dtype=np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    edge = np.array([0x00000000, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001,
                     0x00008000, 0x00018000, 0x3F808000, 0x3F818000], dtype=np.uint32)
    allb = np.concatenate([bits, ties, edge])
    f = allb.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f)
    assert np.array_equal(got, want)
    # specials
    L = oracle.lib()
    assert L.lco_f32_to_bf16(float("inf")) == 0x7F80
    assert L.lco_f32_to_bf16(float("-inf")) == 0xFF80
    assert L.lco_f32_to_bf16(float("nan")) == 0x7FC0
    assert L.lco_bf16_to_f32(0x3F80) == 1.0


def test_bf16_nan_stays_nan(oracle):
    """Every fp32 NaN, whatever its sign and payload, becomes a bf16 NaN
    (exponent all ones, mantissa not zero): dropping the low 16 bits would
    turn a NaN whose payload lies only there into an infinity.  Which NaN is
    the reading of this library (the canonical quiet 0x7FC0, on both sides)."""
    pats = np.array([0x7F800001, 0xFF800001, 0x7F80FFFF, 0x7FA00000, 0xFFC00000,
                     0x7FFFFFFF, 0xFFFFFFFF, 0x7FC00001], dtype=np.uint32)
    got = oracle.f32_to_bf16(pats.view(np.float32))
    assert np.all((got & 0x7F80) == 0x7F80) and np.all((got & 0x007F) != 0)
    assert np.all(got == 0x7FC0)


# ------------------------------------------------------ 1-bit compression --

def test_bit_rule_zero_parity(oracle):
    """Signs packed as 0/1; an exact zero becomes +1 on odd and -1 on even
    iterations (Lion Cub page, "What carries the argument" and the
    alternating-sign assumption)."""
    for t in (1, 2, 3, 4, 101, 1000):
        assert oracle.bit(0.5, t) == 1
        assert oracle.bit(-1e-30, t) == 0
        assert oracle.bit(1e-45, t) == 1            # subnormal is not zero
        z = 1 if t % 2 == 1 else 0
        assert oracle.bit(0.0, t) == z
        assert oracle.bit(-0.0, t) == z


@pytest.mark.parametrize("t", [1, 2])
def test_pack_vote_handworked(oracle, t):
    """tests/golden/pack_vote_w4_d8.json: bytes, counts and signs worked by
    hand (W=4, d=8; t=1: zeros -> 1, t=2: zeros -> 0)."""
    gd = golden("pack_vote_w4_d8.json")
    want = gd["steps"][str(t)]
    x = np.zeros((4, 64), dtype=np.float32)
    x[:, :8] = np.array(gd["x"], dtype=np.float32)
    bits = oracle.pack(x, 8, t)
    assert bits.shape == (4, 1)
    assert [int(w) for w in bits[:, 0]] == want["bytes"]
    counts, sign = oracle.vote(bits, 4, 8, t, oracle.TIE_PARITY)
    assert counts.tolist() == want["counts"]
    assert sign.tolist() == want["sign_parity"]
    counts, sign = oracle.vote(bits, 4, 8, t, oracle.TIE_ZERO)
    assert sign.tolist() == want["sign_zero"]


@pytest.mark.parametrize("t", [1, 2])
def test_pack_layout_matches_numpy_packbits(oracle, t):
    """LSB-first little-endian u64 words, bits past d zero: the layout equals
    NumPy's packbits(bitorder='little') of the 0/1 sign vector."""
    rs = np.random.default_rng(7)
    W, d, ld = 3, 200, 256
    x = rs.standard_normal((W, ld)).astype(np.float32)
    x[rs.random((W, ld)) < 0.1] = 0.0
    x[0, 5] = -0.0
    bits = oracle.pack(x, d, t)
    sgn = (x > 0) | ((x == 0) & (t % 2 == 1))
    sgn[:, d:] = False
    want = np.packbits(sgn, axis=1, bitorder="little").view("<u8")
    assert np.array_equal(bits, want)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5])
def test_vote_bruteforce_all_sign_patterns(oracle, W):
    """Every pattern of c in {-1, 0, +1}^W: the vote equals the sign of the
    sum of +-1 votes (zeros voted by parity), a zero sum (a tie) resolved by
    the tie rule.  Computed by +-1 arithmetic, not by counting bits."""
    pats = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=W)), dtype=np.float32)
    for t in (1, 2, 3, 4):
        for tie in (oracle.TIE_PARITY, oracle.TIE_ZERO):
            for a in range(0, len(pats), 64):
                chunk = pats[a:a + 64]
                d = len(chunk)
                x = np.zeros((W, 64), dtype=np.float32)
                x[:, :d] = chunk.T
                bits = oracle.pack(x, d, t)
                counts, sign = oracle.vote(bits, W, d, t, tie)
                for k in range(d):
                    votes = [1 if v > 0 else -1 if v < 0 else (1 if t % 2 else -1)
                             for v in chunk[k]]
                    S = sum(votes)
                    assert counts[k] == votes.count(1)
                    if S != 0:
                        exp = 1 if S > 0 else -1
                    else:
                        exp = 0 if tie == oracle.TIE_ZERO else (1 if t % 2 else -1)
                    assert sign[k] == exp, (W, t, tie, chunk[k])


# ------------------------------------------------- Lion closed forms -------

def _run(oracle, wl, theta, m, g_fn, steps, debug=False):
    out = []
    for t in range(1, steps + 1):
        g = g_fn(t)
        dbg = oracle.step(wl, theta, m, g, t, debug=debug)
        out.append(dbg)
    return out


@pytest.mark.parametrize("agg", ["vote", "l1"])
def test_lion_closed_form_identical_workers(oracle, agg):
    """W identical workers, m0 = 0, constant g: c_1 = (1-b1) g, every worker
    agrees, the global sign is sgn(g) every step, and the recurrence has the
    closed forms theta_t = a^t theta_0 - sgn(g) (1 - a^t) / wd with
    a = 1 - lr*wd, and m_t = (1 - b2^t) g.  On the L1 path every |c| of a
    tensor is equal, so all codes are +-Qmax and the sign is again sgn(g)."""
    W, steps = 4, 10
    sizes = [64, 4096 + 128]
    wl = wls.Workload(name="cf", tensors=[("a", sizes[0]), ("b", sizes[1])], W=W, agg=agg,
                      qbits=4 if agg == "l1" else 0)
    d, ld = wl.d, wl.ld
    rs = np.random.default_rng(3)
    mag = np.where(np.arange(d) < sizes[0], 1e-3, 3e-2)      # equal |g| per tensor
    gv = (mag * np.where(rs.random(d) < 0.5, -1.0, 1.0)).astype(np.float32)
    theta0 = rs.normal(0, 0.02, d).astype(np.float32)
    theta0[:4] = [0.02, -0.02, 0.0, 5.0]
    theta = theta0.copy()
    m = np.zeros((W, ld), np.float32)
    g = np.zeros((W, ld), np.float32)
    g[:, :d] = gv
    _run(oracle, wl, theta, m, lambda t: g, steps)
    lr, wd, b2 = float(np.float32(wl.lr)), float(np.float32(wl.wd)), float(np.float32(wl.beta2))
    a = 1.0 - lr * wd
    s = np.sign(gv.astype(np.float64))
    th_cf = a**steps * theta0.astype(np.float64) - s * (1 - a**steps) / wd
    m_cf = (1 - b2**steps) * gv.astype(np.float64)
    np.testing.assert_allclose(theta, th_cf, rtol=2e-6, atol=1e-9)
    for i in range(W):
        np.testing.assert_allclose(m[i, :d], m_cf, rtol=2e-6)
    # the worked value theta_0 = 0.02, g > 0 after 10 steps of these hyperparameters
    if gv[0] > 0:
        gd = golden("lion_closed_form.json")
        assert abs(theta[0] - gd["theta_10"]) < gd["theta_10_tol"]


def test_vote_single_worker_is_lion(oracle):
    """W = 1: the majority vote of one worker is that worker's sign, so the
    step is plain Lion on c = b1 m + (1-b1) g (no ties for odd W)."""
    wl = one_tensor(128, 1)
    rs = np.random.default_rng(5)
    theta = rs.normal(0, 0.02, 128).astype(np.float32)
    m = np.zeros((1, 128), np.float32)
    m[0] = rs.normal(0, 1e-3, 128).astype(np.float32)
    g = rs.standard_t(3, (1, 128)).astype(np.float32) * np.float32(1e-3)
    c = np.float32(0.9) * m[0] + np.float32(np.float32(1) - np.float32(0.9)) * g[0]
    dbg = oracle.step(wl, theta, m, g, 1, debug=True)
    assert np.array_equal(dbg["sign"], np.where(c > 0, 1, -1).astype(np.int8))


def test_sign_flip_step_closed_form(oracle):
    """Single worker, m_0 = 1, constant g = -0.05.  The momentum follows
    m_t = b2^t (m_0 - g) + g, so c_t = b1 b2^(t-1) (m_0 - g) + g changes sign
    at the first t with b2^(t-1) < -g / (b1 (m_0 - g)).  Before that step the
    update is -lr, after it +lr (plus decay); theta has the geometric-sum
    closed form.  A swapped b1/b2, a swapped (1-b) factor, or a sign error in
    either update moves the flip step or the limits."""
    b1, b2, m0, gval, steps = 0.9, 0.99, 1.0, -0.05, 400
    wl = one_tensor(64, 1, beta1=b1, beta2=b2)
    theta = np.full(64, 0.5, np.float32)
    m = np.full((1, 64), m0, np.float32)
    g = np.full((1, 64), gval, np.float32)
    signs = [int(dbg["sign"][0]) for dbg in _run(oracle, wl, theta, m, lambda t: g, steps,
                                                 debug=True)]
    ratio = -gval / (b1 * (m0 - gval))
    t_flip = 1 + math.floor(math.log(ratio) / math.log(b2)) + 1
    assert signs[: t_flip - 1] == [1] * (t_flip - 1)
    assert signs[t_flip - 1:] == [-1] * (steps - t_flip + 1)
    assert t_flip == golden("lion_closed_form.json")["sign_flip_step"]
    # theta closed form: theta_T = a^T theta_0 - lr * sum_t a^(T-t) s_t
    lr, wd = float(np.float32(1e-4)), float(np.float32(0.1))
    a = 1 - lr * wd
    T = steps
    k = t_flip - 1                                     # steps with s = +1
    pos = sum(a ** (T - t) for t in range(1, k + 1))
    neg = sum(a ** (T - t) for t in range(k + 1, T + 1))
    th = a**T * 0.5 - lr * (pos - neg)
    np.testing.assert_allclose(theta, th, rtol=1e-5)
    mT = b2**T * (m0 - gval) + gval
    np.testing.assert_allclose(m[0], mT, atol=2e-6)


def _f32(hexstr):
    return float(np.array([int(hexstr, 16)], np.uint32).view(np.float32)[0])


def fp32_order_theta_run(step, case):
    """One vote step of a single worker with c > 0 (s = +1) on a 64-element
    vector holding the case's theta; returns theta' as fp32 bit patterns."""
    wl = one_tensor(64, 1, lr=_f32(case["lr_hex"]), wd=_f32(case["wd_hex"]))
    theta = np.full(64, _f32(case["theta_hex"]), np.float32)
    m = np.zeros((1, wl.ld), np.float32)
    g = np.zeros((1, wl.ld), np.float32)
    g[:, :64] = 1.0                      # c = (1 - beta1) > 0 everywhere
    return step(wl, theta, m, g).view(np.uint32)


def fp32_order_average_run(step):
    """One averaging step of three workers (beta2 = 1/2, g = 0) on the
    fixture's two columns; returns m' as fp32 bit patterns [3][2]."""
    case = golden("fp32_order.json")["average_case"]
    wl = wls.Workload(name="avgorder", tensors=[("wte", 64)], W=case["W"], beta2=case["beta2"],
                      sync_names=("wte",), sync_every=1)
    m = np.zeros((wl.W, wl.ld), np.float32)
    m[:, :2] = np.array(case["m"], np.float32)
    g = np.zeros((wl.W, wl.ld), np.float32)
    return step(wl, None, m, g, want_m=True)[:, :2].view(np.uint32)


def test_fp32_evaluation_order_handworked(oracle):
    """The written order of theta' = theta - (lr*(s + wd*theta)) with one
    rounding per operation and no fused multiply-add, and the worker-order
    fp32 sum of the averaged momenta divided by W, against values worked by
    hand where another order or a contraction would round differently
    (tests/golden/fp32_order.json)."""
    gd = golden("fp32_order.json")

    def step(wl, theta, m, g, want_m=False):
        th = theta if theta is not None else np.zeros(wl.d, np.float32)
        oracle.step(wl, th, m, g, 1)
        return m if want_m else th

    for case in gd["theta_cases"]:
        want = int(case["theta_next_hex"], 16)
        for alt in case["alternatives"].values():
            assert int(alt, 16) != want
        assert np.all(fp32_order_theta_run(step, case) == want), case["name"]
    av = gd["average_case"]
    want = [int(h, 16) for h in av["m_next_hex"]]
    got = fp32_order_average_run(step)
    assert np.all(got == np.array(want, np.uint32)[None, :])
    for alt in av["alternatives"].values():
        assert int(alt, 16) not in want


def test_bf16_theta_one_ulp_of_closed_form(oracle):
    """bf16 parameters: the widened value follows the same closed form to
    within one bf16 ulp per step (the step is computed in fp32, then rounded
    once to bf16)."""
    W = 2
    wl = one_tensor(256, W, theta_dtype="bf16", grad_dtype="bf16")
    rs = np.random.default_rng(11)
    th32 = rs.normal(0, 0.5, 256).astype(np.float32)
    from synth.gen import to_bf16_bits
    theta = to_bf16_bits(th32)
    th0 = bf16_bits_to_f32(theta).astype(np.float64)
    m = np.zeros((W, 256), np.float32)
    gv = np.where(rs.random(256) < 0.5, -1e-3, 1e-3).astype(np.float32)
    g = np.tile(to_bf16_bits(gv), (W, 1))
    oracle.step(wl, theta, m, g, 1)
    s = np.sign(gv)
    lr, wd = float(np.float32(1e-4)), float(np.float32(0.1))
    want = th0 - lr * (s + wd * th0)
    got = bf16_bits_to_f32(theta).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(want))) - 7)
    assert np.all(np.abs(got - want) <= ulp * 0.5 + 1e-12)


def bf16_decay_run(step):
    """bf16 parameters, exact by hand: lr = 2^-4, wd = 1, W = 1, m = 0,
    g = (+1e-3, -1e-3) so the signs are (+1, -1):
      theta = 1:  1 - 2^-4 (1 + 1)    = 0.875
      theta = -2: -2 - 2^-4 (-1 - 2)  = -1.8125
    both exact in bf16 (without the wd*theta term: 0.9375 and -1.9375)."""
    from synth.gen import to_bf16_bits
    wl = one_tensor(2, 1, theta_dtype="bf16", grad_dtype="bf16", lr=2.0 ** -4, wd=1.0)
    theta = to_bf16_bits(np.array([1.0, -2.0], np.float32))
    g = np.zeros((1, 64), np.uint16)
    g[0, :2] = to_bf16_bits(np.array([1e-3, -1e-3], np.float32))
    out = step(wl, theta, np.zeros((1, 64), np.float32), g, 1)
    assert bf16_bits_to_f32(out["theta"]).tolist() == [0.875, -1.8125]


def test_bf16_theta_decay_handworked(oracle):
    bf16_decay_run(oracle_step_fn(oracle))


# ------------------------------------------------------ L1 quantisation ----

def _quant_one(oracle, x, n):
    W = 1
    x = np.asarray(x, dtype=np.float32)
    d = x.size
    wl = one_tensor(d, W, agg="l1", qbits=n)
    xx = np.zeros((1, wl.ld), np.float32)
    xx[0, :d] = x
    codes, m1 = oracle.quant_l1(wl, xx)
    return codes[0, :d].tolist(), float(m1[0, 0])


def test_quant_l1_handworked(oracle):
    """tests/golden/eq1_codes.json: Eq. (1) worked by hand, including products
    that land exactly on .5, which pin round-half-to-even against
    round-half-away."""
    for case in golden("eq1_codes.json")["cases"]:
        codes, M = _quant_one(oracle, case["x"], case["n"])
        assert codes == case["codes"], case
        assert abs(M - case["m1"]) <= case["m1_tol"], case
        if "half_away" in case:
            assert codes != case["half_away"]


def _nearest_even(y: Fraction) -> int:
    f = math.floor(y)
    r = y - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_quant_l1_exact_rational(oracle, n):
    """Random dyadic rows: M1 is the exact mean |x| (every partial sum is
    exact), and each code is the integer in [-Qmax, Qmax] nearest to
    Qmax*x/M1 in exact rational arithmetic, ties to even.  Where the exact
    value lies within the fp64 rounding of the scale and product (2^-48
    relative) of a half-integer, either neighbour is accepted."""
    qmax = 2 ** (n - 1) - 1
    rs = np.random.default_rng(100 + n)
    for trial in range(60):
        L = int(rs.integers(1, 40))
        ks = rs.integers(-300, 301, L)
        if trial % 7 == 0:
            ks[rs.integers(0, L)] = 5000                     # a heavy tail value
        x = ks.astype(np.float32) / np.float32(64)
        codes, M = _quant_one(oracle, x, n)
        S = sum(Fraction(int(abs(k)), 64) for k in ks)
        Mx = S / L
        assert M == float(Mx) or (S == 0 and M == 0.0)
        for xv, k, q in zip(x, ks, codes):
            if S == 0:
                assert q == 0
                continue
            y = Fraction(int(k), 64) * qmax / Mx
            want = max(-qmax, min(qmax, _nearest_even(y)))
            if want != q:
                frac = y - math.floor(y)
                near_half = abs(frac - Fraction(1, 2)) <= abs(y) * Fraction(1, 2**48)
                assert near_half and abs(q - want) == 1 and abs(q) <= qmax, (x, y, q, want)


def scale_precision_run(quant):
    """Eq. (1) on the row x = [v, w] (fp32 bits 0x3e042098, 0x405ef701,
    found by a search over rows whose first code sits close to a rounding
    boundary): M1 = (v + w)/2 exactly, and Qmax*v/M1 is 1/2 - 1.65e-8 in
    exact arithmetic, so Q1(v) = 0 at n = 4; a scale Qmax/M1 rounded to fp32
    (relative error up to 2^-24) moves the product above 1/2 and gives 1.
    The expected codes are computed here in exact rational arithmetic.
    `quant(x, n)` returns (codes, M1) of the one-row, one-tensor vector x."""
    x = np.array([0x3E042098, 0x405EF701], dtype=np.uint32).view(np.float32)
    codes, M = quant(x, 4)
    Mx = (Fraction(float(x[0])) + Fraction(float(x[1]))) / 2
    assert M == float(Mx)
    ys = [Fraction(float(v)) * 7 / Mx for v in x]
    assert Fraction(1, 2) - ys[0] > Fraction(1, 2**27)         # near, but not at, 1/2
    want = [max(-7, min(7, _nearest_even(y))) for y in ys]
    assert want == [0, 7]
    assert list(codes) == want


def test_quant_l1_scale_is_not_rounded_to_fp32(oracle):
    scale_precision_run(lambda x, n: _quant_one(oracle, x, n))


def test_quant_l1_invariants(oracle):
    """Q1(2^k x) = Q1(x) (M1 scales with x) and Q1(-x) = -Q1(x)."""
    rs = np.random.default_rng(9)
    x = (rs.standard_t(3, 5000) * 1e-3).astype(np.float32)
    for n in (2, 4, 8):
        base, _ = _quant_one(oracle, x, n)
        for k in (-5, -1, 1, 7):
            sc, _ = _quant_one(oracle, x * np.float32(2.0**k), n)
            assert sc == base
        neg, _ = _quant_one(oracle, -x, n)
        assert neg == [-v for v in base]


# ------------------------------------------------------------- mean |x| ---

@pytest.mark.parametrize("n", [1, 63, 64, 4095, 4096, 4097, 3 * 4096 + 896,
                               70 * 4096 + 13 * 64, 300 * 4096 + 64, 64 * 256 * 4096 + 4096])
def test_m1_exact_when_sums_are_exact(oracle, n):
    """Values on a 2^-10 grid in [-4, 4]: every partial sum is exact in fp64
    whatever the order, so M1 must be the exact mean rounded once (Python's
    Fraction -> float is correctly rounded).  Spans ragged blocks and more
    than 64 blocks (several partials per finalize lane)."""
    rs = np.random.default_rng(n)
    k = rs.integers(-4096, 4097, n)
    x = (k.astype(np.float64) / 1024).astype(np.float32)
    got = oracle.m1(x)
    want = float(Fraction(int(np.abs(k).sum()), 1024 * n))
    assert got == want


@pytest.mark.parametrize("n", [4096, 70 * 4096 + 13 * 64, 600 * 4096 + 320])
def test_m1_within_summation_error_bound(oracle, n):
    """Magnitudes spread over 1e-30..1e30: the fixed-order tree must lie
    within the worst-case bound of its depth from the correctly rounded sum
    (math.fsum), so no element is dropped, doubled or misindexed."""
    rs = np.random.default_rng(n + 1)
    x = (10.0 ** rs.uniform(-30, 30, n) * np.where(rs.random(n) < 0.5, -1, 1)).astype(np.float32)
    exact = math.fsum(np.abs(x.astype(np.float64)).tolist())
    nb = (n + 4095) // 4096
    ng = (nb + 255) // 256
    depth = 2 + 4 + 6 + 2 + 6 + 2 + (ng + 63) // 64 + 6 + 1
    bound = depth * 2.0**-53 * exact * 1.01
    got = oracle.m1(x) * n
    assert abs(got - exact) <= bound
    # dropping one element must violate the bound for the largest element
    j = int(np.argmax(np.abs(x)))
    y = x.copy()
    y[j] = 0
    assert abs(oracle.m1(y) * n - exact) > bound


def _m1_case_row(case):
    """The case's vector: zeros with 2^e at each placed local index."""
    x = np.zeros(case["n"], np.float32)
    for k, e in case["place"]:
        x[k] = np.float32(2.0**e)
    return x


def _m1_expected(S_hex, n):
    """S / n in one correctly rounded division (Fraction -> float rounds once)."""
    return float(Fraction(float.fromhex(S_hex)) / n)


@pytest.mark.parametrize("case", golden("m1_order.json")["cases"], ids=lambda c: c["name"])
def test_m1_order_handworked(oracle, case):
    """The fixed summation tree of M1 at each of its levels (quad pairing,
    rounds in order, wave halving, block nesting, group fold, final lane runs
    and halving, the element-count divisor), against sums worked by hand from
    the written order; each case also states what a different order would
    give, and that value must differ after the division, so a slip at that
    level in the oracle fails here."""
    x = _m1_case_row(case)
    want = _m1_expected(case["S"], case["n"])
    for alt in case["alternatives"].values():
        assert _m1_expected(alt, case["n"]) != want
    assert oracle.m1(x) == want
    # the sign of a value does not enter, and an exact power-of-two scale
    # passes through every level unchanged
    assert oracle.m1(-x) == want
    assert oracle.m1(x * np.float32(0.25)) == want * 0.25


def test_m1_order_per_tensor_and_worker(oracle):
    """The same hand-worked cases laid out as consecutive tensors of one
    vector (local indices count from each tensor's first element) for two
    workers, the second scaled by 2: the standalone quantiser's per-(worker,
    tensor) M1 must equal every case's worked value."""
    cases = [c for c in golden("m1_order.json")["cases"] if c["n"] <= (1 << 20)]
    # the ragged case has a length that is not a multiple of 64: it goes last
    cases.sort(key=lambda c: c["n"] % 64 != 0)
    wl = wls.Workload(name="m1order", tensors=[(c["name"], c["n"]) for c in cases], W=2,
                      agg="l1", qbits=4)
    x = np.zeros((2, wl.ld), np.float32)
    for T, c in enumerate(cases):
        a = wl.offsets[T]
        x[0, a:a + c["n"]] = _m1_case_row(c)
        x[1, a:a + c["n"]] = -2 * _m1_case_row(c)
    _, m1v = oracle.quant_l1(wl, x)
    for T, c in enumerate(cases):
        want = _m1_expected(c["S"], c["n"])
        assert m1v[0, T] == want, c["name"]
        assert m1v[1, T] == 2 * want, c["name"]


def test_m1_block_reads_past_n_as_zero(oracle):
    rs = np.random.default_rng(2)
    for n in (1, 5, 1000, 4095):
        a = rs.standard_normal(n).astype(np.float32)
        pad = np.zeros(4096, np.float32)
        pad[:n] = a
        assert oracle.m1_block(a) == oracle.m1_block(pad)


# ------------------------------------------------ integer sum and sign ----

def test_l1_sum_handworked(oracle):
    """tests/golden/l1_sum_w2_n2.json: W=2, n=2, one 4-element tensor.  With
    b1 = 0.5 and m = 0, c = g/2 exactly and Q1 is scale-free, so the codes
    are those of g:
      w0 = [0.5, -0.5, 1.5, -1.5]: M1 = 1, codes [0, 0, 1, -1]
      w1 = [1, -3, -1, 1]:        M1 = 1.5, codes [1, -1, -1, 1]
    S = [1, -1, 0, 0] -> sign [+1, -1, 0, 0]; a zero sign only decays theta."""
    gd = golden("l1_sum_w2_n2.json")
    wl = one_tensor(4, gd["W"], agg="l1", qbits=gd["n"], beta1=gd["beta1"])
    theta = np.array(gd["theta"], np.float32)
    th0 = theta.copy()
    m = np.zeros((2, 64), np.float32)
    g = np.zeros((2, 64), np.float32)
    g[:, :4] = np.array(gd["g"], np.float32)
    dbg = oracle.step(wl, theta, m, g, 1, debug=True)
    assert dbg["codes"][:, :4].tolist() == gd["codes"]
    assert dbg["sums"].tolist() == gd["sums"]
    assert dbg["sign"].tolist() == gd["sign"]
    a = 1 - float(np.float32(1e-4)) * float(np.float32(0.1))
    np.testing.assert_allclose(theta[2:], a * th0[2:].astype(np.float64), rtol=1e-7)
    assert theta[0] < th0[0] - 9e-5 and theta[1] > th0[1] + 9e-5


def test_l1_sums_are_column_sums_of_codes(oracle):
    wl = wls.Workload(name="s", tensors=[("a", 4096 * 2 + 64), ("b", 192)], W=5, agg="l1",
                      qbits=3)
    rs = np.random.default_rng(4)
    theta = rs.normal(0, 0.02, wl.d).astype(np.float32)
    m = rs.normal(0, 1e-3, (wl.W, wl.ld)).astype(np.float32)
    g = (rs.standard_t(2.5, (wl.W, wl.ld)) * 1e-3).astype(np.float32)
    dbg = oracle.step(wl, theta, m, g, 1, debug=True)
    S = dbg["codes"][:, : wl.d].astype(np.int32).sum(axis=0)
    assert np.array_equal(S, dbg["sums"])
    assert np.array_equal(np.sign(S).astype(np.int8), dbg["sign"])
    assert np.abs(dbg["codes"]).max() <= 3


# --------------------------------------------------- momentum averaging ---

def test_selective_momentum_average(oracle):
    """b2 = 0.5 and small integers make every momentum exact; on averaging
    steps the flagged tensor's rows all equal the exact worker mean, the
    other tensor is untouched relative to a run without averaging, and
    averaging happens only on steps t % sync_every == 0."""
    W = 4
    base = wls.Workload(name="sync", tensors=[("wte", 128), ("h0", 64)], W=W, beta2=0.5,
                        sync_names=("wte",), sync_every=3)
    nosync = base.with_(sync_names=())
    rs = np.random.default_rng(8)
    m0 = rs.integers(-8, 9, (W, base.ld)).astype(np.float32)
    gs = [rs.integers(-8, 9, (W, base.ld)).astype(np.float32) for _ in range(6)]
    th = np.zeros(base.d, np.float32)
    mA, mB = m0.copy(), m0.copy()
    thA, thB = th.copy(), th.copy()
    mexact = [[Fraction(int(v)) for v in row] for row in m0[:, :base.d]]
    for t in range(1, 7):
        oracle.step(base, thA, mA, gs[t - 1], t)
        oracle.step(nosync, thB, mB, gs[t - 1], t)
        for i in range(W):
            for j in range(base.d):
                mexact[i][j] = mexact[i][j] / 2 + Fraction(int(gs[t - 1][i, j])) / 2
        if t % 3 == 0:
            for j in range(128):
                avg = sum(mexact[i][j] for i in range(W)) / W
                for i in range(W):
                    mexact[i][j] = avg
        for i in range(W):
            assert [Fraction(float(v)) for v in mA[i, :base.d]] == mexact[i]
        assert np.array_equal(mA[:, 128:base.d], mB[:, 128:base.d])
        if t % 3 == 0:
            assert np.all(mA[:, :128] == mA[0, :128])
        if t < 3:                      # no averaging yet: identical runs
            assert np.array_equal(mA, mB) and np.array_equal(thA, thB)


# --------------------------------------------- tie rate (statistical) -----

@pytest.mark.parametrize("W", [4, 8, 16])
def test_majority_tie_rate(oracle, W):
    """Lion Cub page (reference note on majority voting): with 4 workers over
    30% of votes tie, fewer with 8.  For iid symmetric c the tie rate is
    C(W, W/2) / 2^W (0.375, 0.273, 0.196); the oracle's counts must match it
    within 5 sigma."""
    d = 1 << 16
    wl = one_tensor(d, W)
    rs = np.random.default_rng(W)
    theta = np.zeros(d, np.float32)
    m = rs.normal(0, 1e-3, (W, d)).astype(np.float32)
    g = (rs.standard_t(3, (W, d)) * 1e-3).astype(np.float32)
    dbg = oracle.step(wl, theta, m, g, 1, debug=True)
    gd = golden("tie_rate.json")
    p = math.comb(W, W // 2) / 2**W
    assert p == gd["closed_form"][str(W)]
    rate = float(np.mean(2 * dbg["counts"].astype(int) == W))
    assert abs(rate - p) < 5 * math.sqrt(p * (1 - p) / d)
    if W == 4:
        assert rate > gd["W4_min_rate"]


# ------------------------------------------------- streaming form ---------

@pytest.mark.parametrize("agg", ["vote", "l1", "linf"])
def test_chunked_step_equals_whole_step(oracle, agg):
    wl = wls.Workload(name="chunk", tensors=[("a", 4096 * 3 + 640), ("b", 64), ("c", 8192)],
                      W=3, agg=agg, qbits=0 if agg == "vote" else 4, sync_names=("b",),
                      grad_dtype="bf16", theta_dtype="bf16")
    from synth import gen
    theta = gen.host_theta(wl)
    m = gen.host_m(wl)
    g = gen.host_g(wl, 1)
    th1, m_1 = theta.copy(), m.copy()
    oracle.step(wl, th1, m_1, g, 2)
    m1v = {"l1": oracle.m1_all, "linf": oracle.minf_all}.get(agg, lambda *a: None)(wl, m, g)
    th2, m_2 = theta.copy(), m.copy()
    edges = [0, 4096, 4096 * 3, wl.offsets[1] + 64, wl.d]
    for j0, j1 in zip(edges[:-1], edges[1:]):
        tc = np.ascontiguousarray(th2[j0:j1])
        mc = np.ascontiguousarray(m_2[:, j0:j1])
        gc = np.ascontiguousarray(g[:, j0:j1])
        oracle.step_range(wl, j0, j1, m1v, tc, mc, gc, 2)
        th2[j0:j1] = tc
        m_2[:, j0:j1] = mc
    assert np.array_equal(th1, th2)
    assert np.array_equal(m_1, m_2)


# ------------------------- receive side and wire formats (worker-sharded) --

def _words_to_bits(w, n):
    return np.unpackbits(np.ascontiguousarray(w).view(np.uint8), bitorder="little")[:n]


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("tie", ["parity", "zero"])
def test_vote_bits_decode_to_vote_sign(oracle, W, tie):
    """The global-sign bit planes decode (zero ? 0 : sign ? +1 : -1) to the
    brute-force-pinned vote sign for every sign pattern, both parities; a
    parity tie sets no zero bit (a 1-bit result carries it); NumPy's
    unpackbits reads the planes."""
    tm = oracle.TIE_ZERO if tie == "zero" else oracle.TIE_PARITY
    pats = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=W)), dtype=np.float32)
    for t in (1, 2):
        for a in range(0, len(pats), 64):
            chunk = pats[a:a + 64]
            d = len(chunk)
            x = np.zeros((W, 64), dtype=np.float32)
            x[:, :d] = chunk.T
            bits = oracle.pack(x, d, t)
            _, sign = oracle.vote(bits, W, d, t, tm)
            sb, zb = oracle.vote_bits(bits, W, d, t, tm)
            pos = _words_to_bits(sb, 64)
            zer = _words_to_bits(zb, 64)
            dec = np.where(zer[:d] == 1, 0, np.where(pos[:d] == 1, 1, -1))
            assert np.array_equal(dec, sign)
            assert not pos[d:].any() and not zer[d:].any()
            assert not (pos & zer).any()                 # bit 1 means +1, and a zero is not +1
            if tm == oracle.TIE_PARITY:
                assert not zer.any()


def oracle_step_fn(oracle):
    """One whole oracle step on copies of the inputs, returning the new state
    and every debug output; the GPU tests pass a function of the same shape
    backed by the library, so the hand-worked checks below run on both."""
    def step(wl, theta, m, g, t):
        theta, m = theta.copy(), m.copy()
        out = oracle.step(wl, theta, m, g.copy(), t, debug=True)
        out.update(theta=theta, m=m)
        return out
    return step


def tie_rule_run(step, t):
    """W = 2 workers with opposite signs at every element tie the vote.
    With TIE_ZERO the applied sign is 0, and with no weight decay theta does
    not move; with TIE_PARITY a tie takes the exact-zero rule, +1 on odd and
    -1 on even steps, so theta moves by -lr or +lr.  The diagnostics count
    each column once as a tie and, under TIE_ZERO, once as a zero sign,
    never as a match or flip: the sum of c is 0 there (c = +-g/2 exactly)."""
    W, d = 2, 200
    g = np.zeros((W, 256), np.float32)
    g[0, :d] = 0.25
    g[1, :d] = -0.25
    theta0 = np.linspace(-1, 1, d).astype(np.float32)
    for tie in ("zero", "parity"):
        wl = wls.flat("tie", d, W=W, beta1=0.5, wd=0.0, lr=2.0 ** -10, tie=tie)
        out = step(wl, theta0, np.zeros((W, 256), np.float32), g, t)
        s = 0 if tie == "zero" else (1 if t % 2 else -1)
        assert np.all(out["sign"] == s), tie
        assert np.array_equal(out["theta"], theta0 - np.float32(2.0 ** -10) * np.float32(s)), tie
        assert out["stats"][0].tolist() == [d, 0, 0, d if tie == "zero" else 0], tie


@pytest.mark.parametrize("t", [1, 2])
def test_step_tie_rule(oracle, t):
    tie_rule_run(oracle_step_fn(oracle), t)


def test_apply_closed_form(oracle):
    """A constant global sign s applied T times: theta_T = a^T theta_0 -
    s (1 - a^T) / wd (s = 0: pure decay a^T theta_0), m_T = (1 - b2^T) g
    from m_0 = 0, independent of the sign."""
    W, d = 3, 256
    wl = wls.flat("ap", d, W=W)
    rs = np.random.default_rng(12)
    theta0 = rs.normal(0, 0.05, d).astype(np.float32)
    theta = theta0.copy()
    m = np.zeros((W, d), np.float32)
    g = rs.normal(0, 1e-2, (W, d)).astype(np.float32)
    s = rs.integers(-1, 2, d)
    sb = np.packbits(s > 0, bitorder="little").view("<u8").copy()
    zb = np.packbits(s == 0, bitorder="little").view("<u8").copy()
    T = 8
    for t in range(1, T + 1):
        oracle.apply(wl, theta, m, g, t, sb, zb)
    lr, wd, b2 = float(np.float32(1e-4)), float(np.float32(0.1)), float(np.float32(0.99))
    a = 1 - lr * wd
    want = a**T * theta0.astype(np.float64) - s * (1 - a**T) / wd
    np.testing.assert_allclose(theta, want, rtol=2e-6, atol=1e-10)
    np.testing.assert_allclose(m, (1 - b2**T) * g.astype(np.float64), rtol=2e-6)


def test_pack_codes_handworked(oracle):
    """tests/golden/pack_codes_n4_n3.json: n = 4: codes [1, -1, 7, -7, 0, 3]
    are the nibbles 1, F, 7, 9, 0, 3 from the least significant end: word
    0x003097F1.  n = 3: element 10 occupies bits 30..32 and straddles words 0
    and 1; code -3 is 0b101 (bits 30, 32)."""
    for case in golden("pack_codes_n4_n3.json")["cases"]:
        c = np.zeros((1, 64), np.int8)
        for j, v in case["codes"].items():
            c[0, int(j)] = v
        w = oracle.pack_codes(c, case["d"], case["n"])
        assert w.shape == (1, 2 * case["n"])
        want = np.zeros(2 * case["n"], np.uint32)
        for k, v in case["words"].items():
            want[int(k)] = v
        assert np.array_equal(w[0].view(np.uint32), want), case


@pytest.mark.parametrize("n", [2, 3, 4, 5, 7, 8])
def test_pack_codes_roundtrip_and_sum(oracle, n):
    """Independent decode with NumPy (unpackbits, n-bit two's complement)
    recovers the codes; unpack_sum equals NumPy's column sums."""
    qmax = 2 ** (n - 1) - 1
    rs = np.random.default_rng(n)
    W, d = 5, 1000
    ld = 1024
    codes = np.zeros((W, ld), np.int8)
    codes[:, :d] = rs.integers(-qmax, qmax + 1, (W, d))
    wire = oracle.pack_codes(codes, d, n)
    assert wire.shape == (W, (ld // 32) * n)
    bits = np.unpackbits(wire.view(np.uint8), axis=1, bitorder="little")
    fields = bits.reshape(W, ld // 32, 32, n)           # group, element, bit
    val = (fields * (1 << np.arange(n))).sum(axis=3).reshape(W, ld)
    val = np.where(val >= 1 << (n - 1), val - (1 << n), val)
    assert np.array_equal(val[:, :d], codes[:, :d]) and not val[:, d:].any()
    sums, sign = oracle.unpack_sum(wire, W, d, ld, n)
    assert np.array_equal(sums, codes[:, :d].astype(np.int32).sum(axis=0))
    assert np.array_equal(sign, np.sign(sums).astype(np.int8))


@pytest.mark.parametrize("n", [2, 4, 8])
def test_unpack_sum_bits_are_the_signs_of_numpy_column_sums(oracle, n):
    """The p-bit receive side as planes: sign bit where NumPy's column sum of
    the codes is > 0, zero bit where it is 0, nothing past d (ld > d + 64
    leaves whole words past d, which must be written as 0)."""
    qmax = 2 ** (n - 1) - 1
    rs = np.random.default_rng(40 + n)
    W, d, ld = 6, 1000, 1152
    codes = np.zeros((W, ld), np.int8)
    codes[:, :d] = rs.integers(-qmax, qmax + 1, (W, d))
    codes[:, 100:164] = 0                              # a word of exact zero sums
    wire = oracle.pack_codes(codes, d, n)
    sb, zb = oracle.unpack_sum_bits(wire, W, d, ld, n)
    col = codes[:, :d].astype(np.int64).sum(axis=0)
    want_s = np.zeros(ld, np.uint8)
    want_z = np.zeros(ld, np.uint8)
    want_s[:d] = col > 0
    want_z[:d] = col == 0
    assert np.array_equal(_words_to_bits(sb, ld), want_s)
    assert np.array_equal(_words_to_bits(zb, ld), want_z)
    sb2, none = oracle.unpack_sum_bits(wire, W, d, ld, n, zero=False)
    assert none is None and np.array_equal(sb2, sb)


@pytest.mark.parametrize("agg", ["l1"])
def test_p_bit_exchange_composes_into_the_step(oracle, agg):
    """The worker-sharded p-bit flow written out of the oracle's own pieces
    -- quantise each worker's c (quant_l1), pack the codes, unpack and sum
    them into sign and zero planes, apply -- gives theta and m bit for bit
    equal to the fused L1 step, on two tensors with a ragged end."""
    from synth import gen
    wl = wls.Workload(name="pbx", tensors=[("a", 4096 + 640), ("b", 2048)], W=4, agg=agg,
                      qbits=3)
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    g = gen.host_g(wl, 1)
    t = 2
    th1, m_1 = theta.copy(), m.copy()
    oracle.step(wl, th1, m_1, g, t)
    c = np.zeros((wl.W, wl.ld), np.float32)
    for i in range(wl.W):
        c[i, : wl.d] = oracle.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    codes, _ = oracle.quant_l1(wl, c)
    wire = oracle.pack_codes(codes, wl.d, wl.qbits)
    sb, zb = oracle.unpack_sum_bits(wire, wl.W, wl.d, wl.ld, wl.qbits)
    th2, m_2 = theta.copy(), m.copy()
    oracle.apply(wl, th2, m_2, g, t, sb, zb)
    assert np.array_equal(th1, th2)
    assert np.array_equal(m_1, m_2)


def test_avg_aggregation_values(oracle):
    """D-Lion averaging: the applied update is the mean of the W signs,
    (2v - W)/W correctly rounded to fp32 (Python's Fraction -> float rounds
    correctly; fp32 via NumPy), e.g. 1/3 -> 0.33333334 for W = 3, v = 2.
    With identical workers it is plain Lion (s = +-1, the closed form)."""
    for W in (3, 4, 7):
        pats = np.array(list(itertools.product([-1.0, 1.0], repeat=W)), dtype=np.float32)
        d = len(pats)
        wl = wls.flat("avg", d, W=W, agg="avg", beta1=0.5, lr=1.0, wd=0.0)
        theta = np.zeros(d, np.float32)
        m = np.zeros((W, wl.ld), np.float32)
        g = np.zeros((W, wl.ld), np.float32)
        g[:, :d] = pats.T * 2                      # c = g/2 exactly
        dbg = oracle.step(wl, theta, m, g, 1, debug=True)
        v = (pats > 0).sum(axis=1)
        want = np.array([np.float32(float(Fraction(int(2 * k - W), W))) for k in v])
        assert np.array_equal(theta, -want)        # theta' = 0 - 1*(s + 0)
        assert np.array_equal(dbg["sign"], np.sign(2 * v - W).astype(np.int8))
    assert np.float32(float(Fraction(1, 3))) == np.float32(0.33333334)


# ------------------------------------------------------ diagnostics (f3) --

def test_stats_ties_by_construction(oracle):
    """W = 4, columns built with a known number of +1 signs: the tie counter
    equals the number of columns built with exactly two (both parities)."""
    W = 4
    rs = np.random.default_rng(21)
    npos = rs.integers(0, W + 1, 300)
    d = npos.size
    wl = wls.Workload(name="st", tensors=[("a", 128), ("b", d - 128)], W=W, beta1=0.5)
    g = np.zeros((W, wl.ld), np.float32)
    for j, k in enumerate(npos):
        col = np.array([1.0] * k + [-1.0] * (W - k), np.float32)
        g[:, j] = rs.permutation(col)
    for t in (1, 2):
        theta = np.zeros(d, np.float32)
        m = np.zeros((W, wl.ld), np.float32)
        dbg = oracle.step(wl, theta, m, g, t, debug=True)
        assert dbg["stats"][0, 0] == np.count_nonzero(npos[:128] == 2)
        assert dbg["stats"][1, 0] == np.count_nonzero(npos[128:] == 2)
        # with the parity tie rule no applied sign is 0, and sgn(sum c) = sgn(2k - W)
        assert dbg["stats"][:, 3].sum() == 0
        assert dbg["stats"][:, 1].sum() == np.count_nonzero(npos != 2)


def test_stats_match_flip_handworked(oracle):
    """W = 3, n = 2, one tensor of 4 elements, c = g/2 (beta1 = 0.5, m = 0):
      w0 = w1 = [0.5, 0.25, 0.25, 0]: M1 = 0.25, codes [1, 1, 1, 0]
      w2 = [-3, 3, 3, 3]:             M1 = 3,    codes [-1, 1, 1, 1]
    sums [1, 3, 3, 1] -> signs all +1; sum of c [-2, 3.5, 3.5, 3] -> column 0
    flips, columns 1-3 match."""
    gd = golden("stats_match_flip.json")
    wl = wls.flat("mf", 4, W=gd["W"], agg="l1", qbits=gd["n"], beta1=gd["beta1"])
    g = np.zeros((3, 64), np.float32)
    g[:, :4] = np.array(gd["c"], np.float32) * 2           # c = g/2 with m = 0
    dbg = oracle.step(wl, np.zeros(4, np.float32), np.zeros((3, 64), np.float32), g, 1, debug=True)
    assert dbg["sums"].tolist() == gd["sums"]
    assert dbg["stats"][0].tolist() == gd["stats_ties_match_flip_zero"]


def test_stats_momentum_variance_exact(oracle):
    """beta2 = 0.5, m = 0 and small-integer gradients make every new momentum
    exact (g/2), and the fp64 sums exact, so the largest inter-worker
    variance per tensor equals the exact population variance."""
    W = 5
    rs = np.random.default_rng(4)
    wl = wls.Workload(name="mv", tensors=[("a", 64), ("b", 192)], W=W, beta2=0.5)
    g = np.zeros((W, wl.ld), np.float32)
    g[:, : wl.d] = rs.integers(-20, 21, (W, wl.d))
    dbg = oracle.step(wl, np.zeros(wl.d, np.float32), np.zeros((W, wl.ld), np.float32), g, 1,
                      debug=True)
    for T, (a, b) in enumerate([(0, 64), (64, 256)]):
        best = Fraction(0)
        for j in range(a, b):
            vals = [Fraction(int(g[i, j]), 2) for i in range(W)]
            mean = sum(vals) / W
            best = max(best, sum((v - mean) ** 2 for v in vals) / W)
        assert dbg["mvar_max"][T] == float(best)


def zero_spread_run(step):
    """W = 64 identical workers: every new momentum of a column is the same
    value, so the inter-worker variance is 0.  Summed in fp64 in worker
    order, 64 squares need more than 53 bits and S2/W - (S1/W)^2 comes out
    as about -1e-15 for many values (0.8125477, fp32 0x3f500321, among
    them); the spread is the variance floored at 0, so its maximum is 0."""
    W, d = 64, 4096
    rs = np.random.default_rng(6)
    wl = wls.flat("mv0", d, W=W, beta2=0.5)
    v = rs.uniform(0.5, 1.0, d).astype(np.float32)
    v[0] = np.array([0x3F500321], np.uint32).view(np.float32)[0]
    g = np.tile(np.float32(2) * v, (W, 1))             # m' = g/2 = v exactly (beta2 = 1/2, m = 0)
    out = step(wl, np.zeros(d, np.float32), np.zeros((W, d), np.float32), g, 1)
    assert np.array_equal(out["m"][:, :d], np.tile(v, (W, 1)))
    assert out["mvar_max"][0] == 0.0


def test_stats_identical_momenta_have_zero_spread(oracle):
    zero_spread_run(oracle_step_fn(oracle))


# ----------------------------------- max-norm stochastic baseline (Q-inf) --
# The pages name this quantiser as the baseline Eq. (1) replaces but do not
# print it; the reading pinned here is Eq. (1) with max |x| in place of the
# mean and stochastic rounding, u = r * 2^-32 for 32 bits r of a SplitMix64
# output keyed per pair of elements.

def test_splitmix64_published_outputs(oracle):
    """SplitMix64 (Steele, Lea, Flood 2014; Vigna's reference C version):
    the published first outputs for seeds 1234567 and 0."""
    gd = golden("splitmix64.json")
    want = [int(v) for v in gd["seed_1234567_first5"]]
    assert [oracle.splitmix64(1234567, k) for k in range(5)] == want
    assert oracle.splitmix64(0, 0) == int(gd["seed_0_first"])


def test_sr_draws_land_on_published_outputs(oracle):
    """The draw mapping (which SplitMix64 output and which half an element
    takes) against tuples worked by hand to land on the stream's published
    first five outputs: the expected 32 bits are sliced from those published
    values, not recomputed by the generator.  Exercises d, W, t, i, the
    even/odd half and the counter's wrap-around mod 2^64."""
    pub = [int(v) for v in golden("splitmix64.json")["seed_1234567_first5"]]
    gd = golden("sr_draws.json")
    assert gd["seed"] == 1234567
    for tp in gd["tuples"]:
        v = pub[tp["output"]]
        want = v >> 32 if tp["half"] == "high" else v & 0xFFFFFFFF
        got = oracle.sr_u32(gd["seed"], tp["d"], tp["W"], tp["t"], tp["i"], tp["j"])
        assert got == want, tp


def test_minf_is_numpy_max_abs(oracle):
    rs = np.random.default_rng(21)
    for n in (1, 7, 4096, 100003):
        x = (rs.standard_t(2.5, n) * 1e-3).astype(np.float32)
        x[rs.integers(0, n, max(1, n // 50))] = 0
        assert oracle.minf(x) == float(np.max(np.abs(x)))
    x = np.array([0.0, -3.5, 2.0, np.float32(1e-45)], dtype=np.float32)
    assert oracle.minf(x) == 3.5
    assert oracle.minf(np.zeros(5, np.float32)) == 0.0


def _exact_minf(qmax, e=10):
    """A max |x| with qmax / max|x| = 2^e exactly."""
    return float(Fraction(qmax, 2**e))


@pytest.mark.parametrize("n", [2, 4, 8])
def test_qinf_integer_points_ignore_the_draw(oracle, n):
    """y = qmax * x / max|x| an integer: the code is y whatever the draw."""
    qmax = 2 ** (n - 1) - 1
    M = _exact_minf(qmax)
    for k in range(-qmax, qmax + 1):
        c = float(Fraction(k, 2**10))
        for r in (0, 1 << 31, 2**32 - 1):
            assert oracle.qinf(c, M, n, r) == k
    assert oracle.qinf(0.25, 0.0, n, 2**32 - 1) == 0      # all-zero row


def test_qinf_clamps_the_row_maximum(oracle):
    """x = +-max|x| where the fp64 product qmax/M * M rounds above qmax
    (M = float32(0.0066045928), y = 7 + 2^-50): random bits 0 would round up
    to 8, the clamp keeps +-qmax."""
    M = float(np.float32(0.006604592781513929))
    assert M * (7.0 / M) > 7.0
    for r in (0, 2**32 - 1):
        assert oracle.qinf(M, M, 4, r) == 7
        assert oracle.qinf(-M, M, 4, r) == -7


def test_qinf_draw_threshold_direction(oracle):
    """y = 2.25: the code is 3 exactly when u = r / 2^32 < 0.25 (probability
    0.25 of rounding up), else 2; negatives round toward floor(y) + 1 the
    same way."""
    M = _exact_minf(7)
    c = float(Fraction(9, 4 * 2**10))                        # y = 2.25
    at = 1 << 30                                             # u = 0.25
    below = (1 << 30) - 1                                    # u = 0.25 - 2^-32
    assert oracle.qinf(c, M, 4, below) == 3
    assert oracle.qinf(c, M, 4, at) == 2
    assert oracle.qinf(c, M, 4, 0) == 3
    assert oracle.qinf(c, M, 4, 2**32 - 1) == 2
    # y = -2.25 = -3 + 0.75: up to -2 when u < 0.75
    assert oracle.qinf(-c, M, 4, (3 << 30) - 1) == -2
    assert oracle.qinf(-c, M, 4, 3 << 30) == -3
    # a fraction finer than 2^-32: y = 2^-40 rounds up only for r = 0
    c2 = 2.0**-50
    assert oracle.qinf(c2, M, 4, 0) == 1 and oracle.qinf(c2, M, 4, 1) == 0
    # -2^-40 = -1 + (1 - 2^-40): down to -1 needs u >= 1 - 2^-40, which no
    # 32-bit r reaches (the rounding's bias is below 2^-32)
    assert oracle.qinf(-c2, M, 4, 2**32 - 1) == 0 and oracle.qinf(-c2, M, 4, 0) == 0


def test_qinf_unbiased_over_the_stream(oracle):
    """Stochastic rounding is unbiased: over many draws of the generator the
    mean code is y (within 5 standard errors of the Bernoulli mean)."""
    M = _exact_minf(7)
    N = 40000
    for yq in (Fraction(13, 10), Fraction(-5, 8), Fraction(61, 10)):
        c = np.float32(float(yq / 2**10))
        y = Fraction(float(c)) * 2**10                       # the exact y
        qs = np.array([oracle.qinf(float(c), M, 4, oracle.sr_u32(99, N, 1, 0, 0, k))
                       for k in range(N)])
        fl = math.floor(y)
        assert set(np.unique(qs)) <= {fl, fl + 1}
        p = float(y - fl)
        se = math.sqrt(p * (1 - p) / N)
        assert abs(float(np.mean(qs)) - float(y)) < 5 * se + 1e-12


def test_quant_linf_rows_and_counters(oracle):
    """Standalone codes: per (worker, tensor) max |x| exact; element j of
    worker i at step t takes the low (even j) or high (odd j) 32 bits of
    output (t*W + i)*d + 2*floor(j/2) of the seeded stream; the dequantised
    codes are unbiased for x."""
    wl = wls.Workload(name="qi", tensors=[("a", 4096 + 64), ("b", 192)], W=3, agg="linf",
                      qbits=4)
    rs = np.random.default_rng(8)
    x = np.zeros((wl.W, wl.ld), np.float32)
    x[:, : wl.d] = (rs.standard_t(2.5, (wl.W, wl.d)) * 1e-3).astype(np.float32)
    t = 5
    codes, mv = oracle.quant_linf(wl, x, t)
    for i in range(wl.W):
        for T in range(2):
            a, b = wl.offsets[T], wl.offsets[T + 1]
            assert mv[i, T] == float(np.max(np.abs(x[i, a:b])))
    for i, j in ((0, 0), (0, 1), (2, 4100), (2, 4101), (1, wl.d - 1)):
        T = 0 if j < wl.offsets[1] else 1
        r64 = oracle.splitmix64(wl.sr_seed, (t * wl.W + i) * wl.d + (j & ~1))
        r = r64 >> 32 if j & 1 else r64 & 0xFFFFFFFF
        assert oracle.sr_u32(wl.sr_seed, wl.d, wl.W, t, i, j) == r
        assert codes[i, j] == oracle.qinf(float(x[i, j]), mv[i, T], 4, r)
    assert np.all(codes[:, wl.d:] == 0)
    # another step draws a different stream
    codes2, _ = oracle.quant_linf(wl, x, t + 1)
    assert not np.array_equal(codes, codes2)
    # unbiased over steps: mean of dequantised codes tends to x
    acc = np.zeros((wl.W, wl.d))
    S = 200
    for s in range(1, S + 1):
        cs, mv = oracle.quant_linf(wl, x, s)
        scale = np.repeat(mv / 7.0, np.diff(wl.offsets), axis=1)
        acc += cs[:, : wl.d] * scale
    err = acc / S - x[:, : wl.d]
    sd = np.repeat(mv / 7.0, np.diff(wl.offsets), axis=1) * 0.5 / math.sqrt(S)
    assert np.all(np.abs(err) <= 6 * sd + 1e-12)


def test_qinf_zeroes_most_heavy_tailed_updates(oracle):
    """The pages' finding (Lion Cub review, Figure 3 and Figure 4): on
    heavy-tailed update vectors the max-norm quantiser sends most entries to
    zero and matches few signs, while Eq. (1) keeps most signs."""
    gd = golden("q_inf_heavy_tail.json")
    rs = np.random.default_rng(5)
    d = 1 << 18
    wl = wls.flat("ht", d, W=1, agg="linf", qbits=gd["n"])
    x = np.zeros((1, wl.ld), np.float32)
    x[0, :d] = (rs.standard_t(gd["student_t_nu"], d) * 1e-3).astype(np.float32)
    ci, _ = oracle.quant_linf(wl, x, 1)
    c1, _ = oracle.quant_l1(wl.with_(agg="l1"), x)
    zi, z1 = np.mean(ci[0, :d] == 0), np.mean(c1[0, :d] == 0)
    mi = np.mean(np.sign(ci[0, :d]) == np.sign(x[0, :d]))
    m1 = np.mean(np.sign(c1[0, :d]) == np.sign(x[0, :d]))
    assert zi > gd["q_inf_zero_fraction_min"] and z1 < gd["l1_zero_fraction_max"]
    assert m1 > mi + gd["l1_minus_q_inf_match_min"]


def test_linf_step_equals_vote_when_magnitudes_are_equal(oracle):
    """|c| the same everywhere in a row: every code is +-qmax, the integer
    sum is qmax*(2*count - W), and with odd W and no zeros the step is the
    majority-vote step bit for bit."""
    from synth import gen
    wl_v = wls.Workload(name="eq", tensors=[("a", 4096 + 128), ("b", 64)], W=5, agg="vote")
    wl_i = wl_v.with_(agg="linf", qbits=4)
    rs = np.random.default_rng(3)
    theta = gen.host_theta(wl_v)
    m = np.zeros((wl_v.W, wl_v.ld), np.float32)
    g = np.zeros((wl_v.W, wl_v.ld), np.float32)
    g[:, : wl_v.d] = np.where(rs.random((wl_v.W, wl_v.d)) < 0.5, -1.0, 1.0) * 2.0**-9
    tv, mvv = theta.copy(), m.copy()
    dv = oracle.step(wl_v, tv, mvv, g, 3, debug=True)
    ti, mii = theta.copy(), m.copy()
    di = oracle.step(wl_i, ti, mii, g, 3, debug=True)
    assert np.array_equal(np.abs(di["codes"][:, : wl_v.d]), np.full((wl_v.W, wl_v.d), 7))
    assert np.array_equal(di["sums"], 7 * (2 * dv["counts"].astype(np.int32) - wl_v.W))
    assert np.array_equal(di["sign"], dv["sign"])
    assert np.array_equal(ti, tv) and np.array_equal(mii, mvv)
    assert di["stats"][:, 0].sum() == 0                      # no vote ties on this path


def test_linf_step_codes_are_standalone_codes_of_c(oracle):
    """Inside the step, worker i's codes are the standalone max-norm codes of
    its c_i at the same step t (same max |c| per tensor, same draws)."""
    from synth import gen
    wl = wls.Workload(name="sc", tensors=[("a", 4096 + 640), ("b", 128)], W=3, agg="linf",
                      qbits=4, grad_dtype="bf16")
    theta = gen.host_theta(wl)
    m = gen.host_m(wl)
    g = gen.host_g(wl, 4)
    c = np.zeros((wl.W, wl.ld), np.float32)
    for i in range(wl.W):
        c[i, : wl.d] = oracle.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    want, mv = oracle.quant_linf(wl, c, 4)
    assert np.array_equal(mv, oracle.minf_all(wl, m, g))
    got = oracle.step(wl, theta, m.copy(), g, 4, debug=True)
    assert np.array_equal(got["codes"][:, : wl.d], want[:, : wl.d])
    assert np.array_equal(got["sums"], want[:, : wl.d].astype(np.int32).sum(axis=0))
