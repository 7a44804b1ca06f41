"""Shared GPU-test machinery: run the gfx950 library and the CPU oracle on the
same seeded inputs and compare every output.

Bar: bit-exact for bitmaps, vote counts, codes, integer sums and signs; fp32
theta and m within relative 1e-6 and bf16 theta within one bf16 ulp -- and,
since both sides evaluate the same IEEE operations in the same order, bit for
bit as well (checked separately, so a violation of either is reported
distinctly).
"""
import numpy as np

from oracle import lco
from synth import gen


def lioncub_for(wl, **over):
    from communication_compressed_distributed_amd import LionCub
    kw = dict(d=wl.d, W=wl.W, tensor_offsets=wl.offsets, ld=wl.ld,
              sync_m=wl.sync_flags if any(wl.sync_flags) else None, sync_every=wl.sync_every,
              theta_dtype=wl.theta_dtype, grad_dtype=wl.grad_dtype, agg=wl.agg,
              qbits=wl.qbits, tie=wl.tie, beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, wd=wl.wd,
              sr_seed=wl.sr_seed)
    kw.update(over)
    return LionCub(**kw)


def to_dev(a, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_float_state(name, got, want, bf16=False):
    """Tolerance first (the stated bar), then bit equality."""
    if bf16:
        g = got.astype(np.int64)
        w = want.astype(np.int64)
        # one ulp in bf16 is one step of the bit pattern within a binade
        ulps = np.abs(np.where(g >= 0x8000, 0x8000 - g, g) - np.where(w >= 0x8000, 0x8000 - w, w))
        assert ulps.max(initial=0) <= 1, f"{name}: bf16 differs by {ulps.max()} ulp"
        nbad = int(np.count_nonzero(got != want))
        assert nbad == 0, f"{name}: {nbad} bf16 values within 1 ulp but not bit-equal"
        return
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    rel = np.abs(g - w) / np.maximum(np.abs(w), 1e-30)
    bad = rel > 1e-6
    assert not bad.any(), f"{name}: {bad.sum()} values beyond rel 1e-6 (max {rel.max():.3g})"
    nbad = int(np.count_nonzero(bits32(got) != bits32(want)))
    assert nbad == 0, f"{name}: {nbad} values within rel 1e-6 but not bit-equal"


def inject_zeros(wl, m, g, rs, frac=0.01):
    """Zero m and g at random (worker, element) spots so that c is exactly 0
    there (the parity rule), and all workers of some columns (ties at every
    W), and one whole (worker, tensor) row on the quantised paths (norm 0).
    Applies them to the host arrays and returns the positions, so the same
    zeros can be written into the device momentum without copying state."""
    d = wl.d
    mask = rs.random((wl.W, d)) < frac
    m[:, :d][mask] = 0
    g[:, :d][mask] = 0
    cols = rs.integers(0, d, max(1, d // 200))
    m[:, cols] = 0
    g[:, cols] = 0
    row = None
    if wl.agg in ("l1", "linf") and wl.n_tensors > 1:
        a, b = wl.offsets[1], wl.offsets[2]
        m[wl.W - 1, a:b] = 0
        g[wl.W - 1, a:b] = 0
        row = (wl.W - 1, a, b)
    return mask, cols, row


def zero_device_m(d_m, wl, zeros):
    """Write the zeros inject_zeros chose into the device momentum in place:
    the device keeps its own trajectory (nothing of the oracle's state is
    copied over), only the same inputs are perturbed on both sides."""
    import torch
    mask, cols, row = zeros
    view = d_m[:, : wl.d]
    view[torch.from_numpy(mask).to(d_m.device)] = 0
    d_m[:, torch.from_numpy(cols).to(d_m.device)] = 0
    if row is not None:
        i, a, b = row
        d_m[i, a:b] = 0


def gpu_step_fn():
    """One library step on device copies of host inputs, returning the new
    state and every debug output as host arrays (the same keys as the
    oracle's step), so a hand-worked check can run on the library directly."""
    import torch

    def step(wl, theta, m, g, t):
        tb, gb = wl.theta_dtype == "bf16", wl.grad_dtype == "bf16"
        lc = lioncub_for(wl.with_(ld_pad=m.shape[1] - wl.ld))
        d_theta, d_m, d_g = to_dev(theta, tb), to_dev(m), to_dev(g, gb)
        dbg = {"sign": torch.zeros(wl.d, dtype=torch.int8, device="cuda"),
               "stats": torch.full((wl.n_tensors, 4), -1, dtype=torch.int64, device="cuda"),
               "mvar_max": torch.full((wl.n_tensors,), -1.0, dtype=torch.float64, device="cuda")}
        if wl.agg in ("vote", "avg"):
            dbg["bits"] = torch.full((wl.W, m.shape[1] // 64), -1, dtype=torch.int64, device="cuda")
            dbg["counts"] = torch.zeros(wl.d, dtype=torch.uint8, device="cuda")
        else:
            dbg["codes"] = torch.zeros((wl.W, m.shape[1]), dtype=torch.int8, device="cuda")
            dbg["sums"] = torch.zeros(wl.d, dtype=torch.int32, device="cuda")
            dbg["m1"] = torch.zeros((wl.W, wl.n_tensors), dtype=torch.float64, device="cuda")
        lc.step(d_theta, d_m, d_g, t, dbg)
        torch.cuda.synchronize()
        lc.close()
        out = {k: to_host(v) for k, v in dbg.items()}
        out["stats"] = out["stats"].view(np.uint64)
        if "bits" in out:
            out["bits"] = out["bits"].view(np.uint64)
        out["theta"] = to_host(d_theta)
        if tb:
            out["theta"] = out["theta"].view(np.uint16)
        out["m"] = to_host(d_m)
        return out
    return step


def gpu_step_vs_oracle(wl, steps=2, t0=1, zeros=True, debug=True, seed_shift=0):
    """Run `steps` steps on both sides from the same seeded state; compare
    everything after every step.  Each side carries its own theta and m from
    step to step (independent trajectories: the device state is never reset
    from the oracle's).  Returns a small summary dict."""
    import torch
    rs = np.random.default_rng(1234 + seed_shift)
    theta = gen.host_theta(wl)
    m = gen.host_m(wl)
    tb, gb = wl.theta_dtype == "bf16", wl.grad_dtype == "bf16"
    lc = lioncub_for(wl)
    d_theta = to_dev(theta, tb)
    d_m = to_dev(m)
    ties = 0
    for t in range(t0, t0 + steps):
        g = gen.host_g(wl, t)
        if zeros:
            zero_device_m(d_m, wl, inject_zeros(wl, m, g, rs))
        d_g = to_dev(g, gb)
        dbg = None
        if debug:
            dbg = {"sign": torch.zeros(wl.d, dtype=torch.int8, device="cuda"),
                   "stats": torch.full((wl.n_tensors, 4), -1, dtype=torch.int64, device="cuda"),
                   "mvar_max": torch.full((wl.n_tensors,), -1.0, dtype=torch.float64,
                                          device="cuda")}
            if wl.agg in ("vote", "avg"):
                dbg["bits"] = torch.full((wl.W, wl.ld // 64), -1, dtype=torch.int64, device="cuda")
                dbg["counts"] = torch.zeros(wl.d, dtype=torch.uint8, device="cuda")
            else:
                dbg["codes"] = torch.zeros((wl.W, wl.ld), dtype=torch.int8, device="cuda")
                dbg["sums"] = torch.zeros(wl.d, dtype=torch.int32, device="cuda")
        lc.step(d_theta, d_m, d_g, t, dbg)
        torch.cuda.synchronize()
        want = lco.step(wl, theta, m, g, t, debug=debug)
        check_float_state(f"theta t={t}", to_host(d_theta), theta, bf16=tb)
        check_float_state(f"m t={t}", to_host(d_m)[:, : wl.d], m[:, : wl.d])
        if debug:
            got_sign = to_host(dbg["sign"])
            if wl.agg in ("vote", "avg"):
                gb_ = to_host(dbg["bits"]).view(np.uint64)
                assert np.array_equal(gb_, want["bits"]), f"bits t={t}"
                gc = to_host(dbg["counts"])
                assert np.array_equal(gc, want["counts"]), f"counts t={t}"
                ties += int(np.count_nonzero(2 * gc.astype(int) == wl.W))
            else:
                assert np.array_equal(to_host(dbg["codes"])[:, : wl.d],
                                      want["codes"][:, : wl.d]), f"codes t={t}"
                assert np.array_equal(to_host(dbg["sums"]), want["sums"]), f"sums t={t}"
            assert np.array_equal(got_sign, want["sign"]), f"sign t={t}"
            assert np.array_equal(to_host(dbg["stats"]).view(np.uint64), want["stats"]), \
                f"stats t={t}: {to_host(dbg['stats'])} vs {want['stats']}"
            assert np.array_equal(to_host(dbg["mvar_max"]).view(np.uint64),
                                  want["mvar_max"].view(np.uint64)), f"mvar_max t={t}"
    lc.close()
    return {"d": wl.d, "W": wl.W, "steps": steps, "ties": ties, "ok": True}
