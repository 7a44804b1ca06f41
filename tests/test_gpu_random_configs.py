"""Seeded random configurations against the oracle: tensor splits (64-aligned
offsets, tensors from 64 elements to several 4096-element blocks with ragged
ends), worker counts 1..40, every aggregation mode, code widths 2..8, both
tie rules, fp32/bf16 theta and gradients, momentum sync on random tensors
and intervals, row padding, random step indices.  Each configuration runs
two steps with the debug outputs and one production step; everything is
compared bit for bit."""
import os

import numpy as np
import pytest

from oracle import lco
from synth import gen
from synth import workloads as wls
from tests.harness import gpu_step_vs_oracle

pytestmark = pytest.mark.gpu

# configurations k = FIRST .. FIRST + N - 1 (the environment can widen the
# sweep for a longer run; the default suite runs the first 100)
N_CONFIGS = int(os.environ.get("LIONCUB_RANDOM_CONFIGS", "100"))
FIRST_CONFIG = int(os.environ.get("LIONCUB_RANDOM_FIRST", "0"))


def random_workload(k):
    rs = np.random.default_rng(1000 + k)
    n_t = int(rs.integers(1, 7))
    tensors = []
    for T in range(n_t):
        kind = rs.integers(0, 3)
        if kind == 0:
            n = 64 * int(rs.integers(1, 20))                  # small, 64-multiple
        elif kind == 1:
            n = 4096 * int(rs.integers(1, 4))                 # whole blocks
        else:
            n = 4096 * int(rs.integers(0, 4)) + 64 * int(rs.integers(1, 64))
        tensors.append((f"t{T}", n))
    last = tensors[-1]
    tensors[-1] = (last[0], last[1] + int(rs.integers(0, 64)))  # ragged end of d
    agg = ["vote", "avg", "l1", "linf"][int(rs.integers(0, 4))]
    W = int(rs.integers(1, 41))
    sync = tuple(nm for nm, _ in tensors if rs.random() < 0.3)
    return wls.Workload(
        name=f"rand{k}", tensors=tensors, W=W, agg=agg,
        qbits=0 if agg in ("vote", "avg") else int(rs.integers(2, 9)),
        tie=["parity", "zero"][int(rs.integers(0, 2))],
        theta_dtype=["f32", "bf16"][int(rs.integers(0, 2))],
        grad_dtype=["f32", "bf16"][int(rs.integers(0, 2))],
        sync_names=sync, sync_every=int(rs.integers(1, 4)),
        ld_pad=64 * int(rs.integers(0, 3)), seed=k, sr_seed=int(rs.integers(0, 2**63)),
        g_tensor_scale=(1e-4, 1e-2) if rs.random() < 0.5 else None)


@pytest.mark.parametrize("k", range(FIRST_CONFIG, FIRST_CONFIG + N_CONFIGS))
def test_random_config(k):
    wl = random_workload(k)
    t0 = int(np.random.default_rng(k).integers(1, 1000))
    print(wl.name, wl.agg, "W", wl.W, "n", wl.qbits, "tensors", [n for _, n in wl.tensors],
          wl.theta_dtype, wl.grad_dtype, "sync", wl.sync_names, wl.sync_every, "t0", t0,
          flush=True)
    gpu_step_vs_oracle(wl, steps=2, t0=t0, debug=True)
    gpu_step_vs_oracle(wl, steps=1, t0=t0 + 2, debug=False, seed_shift=1)


def random_hyper_workload(k):
    """A random configuration as above with random hyperparameters and value
    scales, including the degenerate ones: beta1 = 1 (c = m) or 0 (c = g),
    beta2 = 1 (m' = m) or 0 (m' = g), lr = 0 (theta unchanged), wd = 0 or
    large, and parameters, momenta and gradients from 1e-30 (subnormal
    products) to 1e3."""
    rs = np.random.default_rng(7000 + k)
    pick = lambda xs: xs[int(rs.integers(0, len(xs)))]
    return random_workload(k).with_(
        name=f"hyper{k}",
        beta1=pick([0.9, 0.5, 0.0, 1.0, float(np.float32(rs.random()))]),
        beta2=pick([0.99, 0.95, 0.0, 1.0, float(np.float32(rs.random()))]),
        lr=pick([1e-4, 1e-2, 0.5, 0.0, float(np.float32(rs.random() * 1e-3))]),
        wd=pick([0.1, 0.0, 1.0, float(np.float32(rs.random()))]),
        theta_std=pick([0.02, 1e3, 1e-20]),
        m_std=pick([1e-3, 1.0, 1e-30]),
        g_scale=pick([1e-3, 1e2, 1e-30]),
        g_tensor_scale=None)


N_HYPER = int(os.environ.get("LIONCUB_RANDOM_HYPER", "60"))


@pytest.mark.parametrize("k", range(N_HYPER))
def test_random_hyperparameters(k):
    wl = random_hyper_workload(k)
    t0 = int(np.random.default_rng(50_000 + k).integers(1, 1000))
    print(wl.name, wl.agg, "W", wl.W, "n", wl.qbits, "beta", wl.beta1, wl.beta2, "lr", wl.lr,
          "wd", wl.wd, "scales", wl.theta_std, wl.m_std, wl.g_scale, "t0", t0, flush=True)
    gpu_step_vs_oracle(wl, steps=2, t0=t0, debug=True)
    gpu_step_vs_oracle(wl, steps=1, t0=t0 + 2, debug=False, seed_shift=1)


N_EXCHANGE = 40


@pytest.mark.parametrize("k", range(N_EXCHANGE))
def test_random_config_exchange_composes_into_the_step(k):
    """On the same random configurations, the worker-sharded exchange built
    from the standalone calls -- vote path: pack(c) -> vote_bits; quantised
    paths: quant_l1 / quant_linf(c) -> pack_codes -> unpack_sum_bits; then
    apply -- leaves theta and m bit for bit where the fused step leaves
    them.  The averaging path applies fractional signs and has no planes."""
    import torch
    from tests.harness import lioncub_for, to_dev
    wl = random_workload(k)
    if wl.agg == "avg":
        pytest.skip("the averaging path has no sign planes")
    t = int(np.random.default_rng(k).integers(1, 1000))
    tb, gb = wl.theta_dtype == "bf16", wl.grad_dtype == "bf16"
    theta, m = gen.host_theta(wl), gen.host_m(wl)
    g = gen.host_g(wl, t)
    c = np.zeros((wl.W, wl.ld), np.float32)
    for i in range(wl.W):
        c[i, : wl.d] = lco.c_row(wl, m[i, : wl.d], g[i, : wl.d])
    lc = lioncub_for(wl)
    dg = to_dev(g, gb)
    thA, mA = to_dev(theta, tb), to_dev(m)
    lc.step(thA, mA, dg, t)
    words = wl.ld // 64
    sb = torch.empty(words, dtype=torch.int64, device="cuda")
    zb = torch.empty(words, dtype=torch.int64, device="cuda")
    if wl.agg == "vote":
        bits = torch.empty((wl.W, words), dtype=torch.int64, device="cuda")
        lc.pack(to_dev(c), t, bits)
        lc.vote_bits(bits, t, sb, zb)
    else:
        codes = torch.empty((wl.W, wl.ld), dtype=torch.int8, device="cuda")
        if wl.agg == "l1":
            lc.quant_l1(to_dev(c), codes)
        else:
            lc.quant_linf(to_dev(c), t, codes)
        wire = torch.empty((wl.W, (wl.ld // 32) * wl.qbits), dtype=torch.int32, device="cuda")
        lc.pack_codes(codes, wire)
        lc.unpack_sum_bits(wire, sb, zb)
    thB, mB = to_dev(theta, tb), to_dev(m)
    lc.apply(thB, mB, dg, t, sb, zb)
    torch.cuda.synchronize()
    assert torch.equal(thA.view(torch.int16) if tb else thA, thB.view(torch.int16) if tb else thB)
    assert torch.equal(mA[:, : wl.d], mB[:, : wl.d])
    lc.close()
