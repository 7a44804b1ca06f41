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
