"""Seeded random configurations against the oracle: tensor splits (64-aligned
offsets, tensors from 64 elements to several 4096-element blocks with ragged
ends), worker counts 1..40, every aggregation mode, code widths 2..8, both
tie rules, fp32/bf16 theta and gradients, momentum sync on random tensors
and intervals, row padding, random step indices.  Each configuration runs
two steps with the debug outputs and one production step; everything is
compared bit for bit."""
import numpy as np
import pytest

from synth import workloads as wls
from tests.harness import gpu_step_vs_oracle

pytestmark = pytest.mark.gpu

N_CONFIGS = 100


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


@pytest.mark.parametrize("k", range(N_CONFIGS))
def test_random_config(k):
    wl = random_workload(k)
    t0 = int(np.random.default_rng(k).integers(1, 1000))
    print(wl.name, wl.agg, "W", wl.W, "n", wl.qbits, "tensors", [n for _, n in wl.tensors],
          wl.theta_dtype, wl.grad_dtype, "sync", wl.sync_names, wl.sync_every, "t0", t0,
          flush=True)
    gpu_step_vs_oracle(wl, steps=2, t0=t0, debug=True)
    gpu_step_vs_oracle(wl, steps=1, t0=t0 + 2, debug=False, seed_shift=1)
