"""bench.py's host logic (no GPU): the multi-threaded CPU baseline runs the
oracle's serial routine on disjoint column ranges and must give exactly the
whole-array step."""
import numpy as np
import pytest

import bench
from synth import gen
from synth import workloads as wls


@pytest.mark.parametrize("agg,qbits,gdt", [("vote", 0, "f32"), ("avg", 0, "bf16"),
                                           ("l1", 4, "f32"), ("l1", 8, "bf16"),
                                           ("linf", 4, "f32")])
@pytest.mark.parametrize("P", [1, 3, 8])
def test_threaded_oracle_step_equals_whole_step(oracle, agg, qbits, gdt, P):
    wl = wls.flat("thr", 5 * 4096 + 200, W=5, agg=agg, qbits=qbits, grad_dtype=gdt,
                  theta_dtype="bf16" if gdt == "bf16" else "f32")
    th, m, g = gen.host_theta(wl), gen.host_m(wl), gen.host_g(wl, 3)
    th1, m1 = th.copy(), m.copy()
    oracle.step(wl, th1, m1, g, 3)
    th2, m2 = th.copy(), m.copy()
    bench.oracle_step_threaded(wl, th2, m2, g, 3, P)
    assert np.array_equal(th1, th2)
    assert np.array_equal(m1, m2)


def test_cpu_threads_is_bounded():
    assert 1 <= bench.cpu_threads() <= 16


def test_gpus_above_one_exit_with_a_message(capsys):
    import sys
    argv = sys.argv
    sys.argv = ["bench.py", "--gpus", "2"]
    try:
        with pytest.raises(SystemExit) as e:
            bench.main()
    finally:
        sys.argv = argv
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
