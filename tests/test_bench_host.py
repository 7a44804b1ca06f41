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


def test_cpu_threads_uses_every_allowed_cpu_within_the_quota(monkeypatch):
    import os
    P, host = bench.cpu_threads()
    assert host["host_cpus"] == os.cpu_count()
    assert host["allowed_cpus"] == len(os.sched_getaffinity(0))
    assert 1 <= P <= host["allowed_cpus"]
    if host["cgroup_cpu_quota"] is None:
        assert P == host["allowed_cpus"]
    monkeypatch.setattr(bench, "cpu_quota", lambda: 2.5)
    assert bench.cpu_threads()[0] == min(2, host["allowed_cpus"])
    monkeypatch.setattr(bench, "cpu_quota", lambda: None)
    assert bench.cpu_threads()[0] == host["allowed_cpus"]


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


@pytest.mark.parametrize("name,step_total,fused,norm", [
    ("flat-1M-w4-vote", 56, 56, 0),                          # 4*(4+4+4) + 2*4
    ("gpt2-124M-w8-vote", 104, 104, 0),                      # 8*12 + 8
    ("flat-350M-w16-l1q4", 328, 200, 128),                   # 16*8 + (16*12 + 8)
    ("gpt-760M-w8-vote-bf16-syncemb", 84, 84, 0),            # 8*(4+2+4) + 2*2
    ("gpt-1.3B-w8-l1q8-bf16g", 136, 88, 48),                 # 8*6 + (8*10 + 8)
])
def test_algorithmic_bytes_per_parameter(name, step_total, fused, norm):
    """The roofline's numerator: what the method must move per parameter
    with every intermediate in registers (m and g read and m written once
    per worker, theta read and written once; the quantised paths read m and
    g once more for the norm pass)."""
    wl = wls.BY_NAME[name]
    b = bench.bytes_per_param(wl)
    assert b["step_total"] == step_total
    kind = {"vote": "vote_step", "l1": "l1_step"}[wl.agg]
    assert b[kind] == fused
    assert (b["m1_partial"] if wl.agg == "l1" else 0) == norm
    # the whole step's bytes at the workload's size (GB), as the bench prices it
    assert abs(step_total * wl.d / 1e9 - {"flat-1M-w4-vote": 0.0587, "gpt2-124M-w8-vote": 12.94,
                                         "flat-350M-w16-l1q4": 114.8,
                                         "gpt-760M-w8-vote-bf16-syncemb": 63.73,
                                         "gpt-1.3B-w8-l1q8-bf16g": 178.65}[name]) < 0.01


def test_traffic_digest_ignores_comments_not_code():
    """Editing a comment keeps the HBM-traffic record valid; editing code
    invalidates it."""
    import os
    pkg = os.path.join(bench.ROOT, "communication_compressed_distributed_amd")

    def read(rel, edit=None):
        with open(os.path.join(pkg, rel)) as f:
            text = f.read()
        return edit(text) if edit and rel.endswith("step.hip") else text

    base = bench.kernel_source_digest()
    assert bench.kernel_source_digest(lambda r: read(r, lambda t: t + "\n// a note\n/* and\n more */\n")) == base
    assert bench.kernel_source_digest(lambda r: read(r, lambda t: t.replace("\n", "\n\n  ", 5))) == base
    assert bench.kernel_source_digest(lambda r: read(r, lambda t: t + "\nstatic int x;\n")) != base
