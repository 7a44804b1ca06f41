"""The allocation-free step, lioncub_step_static, against the context step,
lioncub_step, through the C ABI on the same inputs: several calls in a row
on one GPU, each on a smaller or differently shaped configuration than the
one before (so stale tables or partials left in the library's fixed scratch
array would show), bit for bit on theta and m (within the fp32 / bf16 bar
first, then bitwise).  Also a call captured into a HIP graph and replayed."""
import numpy as np
import pytest

from communication_compressed_distributed_amd import _abi
from synth import gen
from synth import workloads as wls
from tests.harness import check_float_state, lioncub_for, to_dev, to_host

pytestmark = pytest.mark.gpu

# Largest first; each later one is smaller or cut differently.
CASES = [
    wls.Workload(name="na-l1-gpt", tensors=wls.shrink(wls.GPT_1B3_W8_L1Q8, 40 * 4096 + 320,
                                                      40).tensors,
                 W=8, agg="l1", qbits=8, grad_dtype="bf16"),
    wls.Workload(name="na-l1-small", tensors=[("a", 9 * 4096 + 64), ("b", 4096), ("c", 832)],
                 W=5, agg="l1", qbits=4, sync_names=("a",), sync_every=2),
    wls.flat("na-vote", 3 * 4096 + 100, W=4, agg="vote", theta_dtype="bf16"),
    # a long list after the short ones: 2,000 tensors, tables in 63 launches
    wls.Workload(name="na-l1-2000", tensors=[(f"t{k}", 64 * (1 + k % 5)) for k in range(2000)],
                 W=3, agg="l1", qbits=3),
]


def _inputs(wl, t):
    return gen.host_theta(wl), gen.host_m(wl), gen.host_g(wl, t)


def _compare_one(wl, t):
    import torch
    theta, m, g = _inputs(wl, t)
    tb, gb = wl.theta_dtype == "bf16", wl.grad_dtype == "bf16"
    # the existing entry point: a context with a torch-allocated workspace
    lc = lioncub_for(wl)
    r_theta, r_m, r_g = to_dev(theta, tb), to_dev(m), to_dev(g, gb)
    lc.step(r_theta, r_m, r_g, t)
    # the allocation-free one on copies of the same inputs
    s_theta, s_m, s_g = to_dev(theta, tb), to_dev(m), to_dev(g, gb)
    stream = torch.cuda.current_stream()
    _abi.lioncub_step_static(lc.cfg, _abi._stream_handle(stream), s_theta, s_m, s_g, t)
    torch.cuda.synchronize()
    check_float_state(f"{wl.name} theta t={t}", to_host(s_theta), to_host(r_theta), bf16=tb)
    check_float_state(f"{wl.name} m t={t}", to_host(s_m)[:, : wl.d], to_host(r_m)[:, : wl.d])
    # columns past d untouched by both
    assert np.array_equal(to_host(s_m)[:, wl.d:], m[:, wl.d:])
    lc.close()


def test_static_step_matches_context_step_calls_in_a_row():
    for t, wl in zip((1, 2, 3, 5), CASES):
        print("no-alloc", wl.name, "d", wl.d, "W", wl.W, "t", t, flush=True)
        _compare_one(wl, t)
    # and back to the first, largest shape after the smaller ones
    print("no-alloc", CASES[0].name, "again", flush=True)
    _compare_one(CASES[0], 4)


def test_static_step_rejects_oversized_config():
    import torch
    wl = wls.flat("na-big", 350_000_000, W=128, agg="l1", qbits=4)
    cfg = _abi.make_config(wl.d, wl.ld, wl.W, wl.offsets, agg=_abi.AGG_L1SUM, qbits=4)
    assert _abi.lioncub_workspace_bytes(cfg) > _abi.STATIC_SCRATCH_BYTES
    x = torch.zeros(64, device="cuda")
    with pytest.raises(_abi.LionCubError) as e:
        _abi.lioncub_step_static(cfg, _abi._stream_handle(), x, x, x, 1)
    assert e.value.status == _abi.ESCRATCH


def test_static_step_in_a_graph():
    """Kernel launches only: the call can be captured; three replays, each
    with eager work of the context step in between, track the context step."""
    import torch
    wl = CASES[1]
    t = 2
    theta, m, g = _inputs(wl, t)
    r_theta, r_m, r_g = to_dev(theta), to_dev(m), to_dev(g)
    s_theta, s_m, s_g = to_dev(theta), to_dev(m), to_dev(g)
    lc = lioncub_for(wl)
    # an eager call first, so the array's address on this device is known
    # before capture starts
    _compare_one(CASES[2], 1)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        _abi.lioncub_step_static(lc.cfg, _abi._stream_handle(side), s_theta, s_m, s_g, t)
    for rep in range(3):
        # another shape through the same scratch array between replays
        _compare_one(CASES[2], 1)
        graph.replay()
        lc.step(r_theta, r_m, r_g, t)
        torch.cuda.synchronize()
        check_float_state(f"graph replay {rep} theta", to_host(s_theta), to_host(r_theta))
        check_float_state(f"graph replay {rep} m", to_host(s_m)[:, : wl.d],
                          to_host(r_m)[:, : wl.d])
    lc.close()


def test_static_step_wrapper_matches_context_step():
    """The checked Python wrapper (StaticStep) over the allocation-free entry
    point, two steps in a row on one state, against LionCub.step."""
    import torch

    from communication_compressed_distributed_amd import StaticStep
    wl = CASES[1]
    theta, m, _ = _inputs(wl, 1)
    lc = lioncub_for(wl)
    st = StaticStep(d=wl.d, W=wl.W, tensor_offsets=wl.offsets, ld=wl.ld,
                    sync_m=wl.sync_flags if any(wl.sync_flags) else None,
                    sync_every=wl.sync_every, theta_dtype=wl.theta_dtype,
                    grad_dtype=wl.grad_dtype, agg=wl.agg, qbits=wl.qbits, tie=wl.tie,
                    beta1=wl.beta1, beta2=wl.beta2, lr=wl.lr, wd=wl.wd, sr_seed=wl.sr_seed)
    r_theta, r_m = to_dev(theta), to_dev(m)
    s_theta, s_m = to_dev(theta), to_dev(m)
    for t in (1, 2):
        g = to_dev(gen.host_g(wl, t))
        lc.step(r_theta, r_m, g, t)
        st.step(s_theta, s_m, g, t)
        torch.cuda.synchronize()
        check_float_state(f"wrapper theta t={t}", to_host(s_theta), to_host(r_theta))
        check_float_state(f"wrapper m t={t}", to_host(s_m)[:, : wl.d], to_host(r_m)[:, : wl.d])
    with pytest.raises(ValueError):
        st.step(s_theta[:-1], s_m, g, 3)
    lc.close()


@pytest.mark.slow
@pytest.mark.parametrize("wl", [wls.GPT_760M_W8_VOTE_SYNC, wls.GPT_1B3_W8_L1Q8],
                         ids=lambda w: w.name)
def test_static_step_full_size_tensor_lists(wl):
    """The two 292-tensor GPT lists at full size (the tables rebuilt in
    several launches of 32 tensor entries every call; the 1.3B list's
    workspace, 44 MiB, is the largest of the workloads): two allocation-free
    steps against two context steps on copies of the same device state,
    theta and m bit-equal after each."""
    import torch
    torch.cuda.set_device(0)
    theta, m = gen.device_theta(wl), gen.device_m(wl)
    g = gen.device_g(wl, 1)
    s_theta, s_m = theta.clone(), m.clone()
    lc = lioncub_for(wl)
    stream = torch.cuda.current_stream()

    def bits(x):
        return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
    for t in (1, 2):
        gen.fill_device_g(wl, t, g)
        lc.step(theta, m, g, t)
        _abi.lioncub_step_static(lc.cfg, _abi._stream_handle(stream), s_theta, s_m, g, t)
        torch.cuda.synchronize()
        assert torch.equal(bits(s_theta), bits(theta)), f"{wl.name} theta t={t}"
        assert torch.equal(bits(s_m), bits(m)), f"{wl.name} m t={t}"
        print("no-alloc full size", wl.name, "t", t, "bit-equal", flush=True)
    lc.close()
    del theta, m, g, s_theta, s_m
    torch.cuda.empty_cache()
