"""AddressSanitizer + UndefinedBehaviorSanitizer over the host code (CPU
only; no GPU code is built with them).

- The oracle (oracle/lco.c) built by gcc with -fsanitize=address,undefined
  and -fno-sanitize-recover, every entry point driven on small inputs in a
  child process (any report aborts it).
- The host side of the library (csrc/lioncub.cpp: configuration checks,
  workspace layout, table building, error paths) compiled with host-only
  sanitizers and linked with the kernel objects build() left in _build/;
  the host ABI tests run against it in a child process.  Skipped when those
  objects are absent (run build() first).
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "communication_compressed_distributed_amd")
OBJ = os.path.join(ROOT, "_build")
KERNEL_OBJS = ["step.hip.o", "l1.hip.o", "bits.hip.o", "wire.hip.o"]
# sources with host code of the C ABI, rebuilt here with host sanitizers
HOST_SRCS = ["lioncub.cpp", "tables.hip", "static.hip"]


def _run_child(code, preload, env_extra=None):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": preload, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    env.update(env_extra or {})
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], capture_output=True,
                          text=True, env=env, timeout=600, cwd=ROOT)


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liblco_san.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-ffp-contract=off", "-fPIC", "-shared", "-o", lib,
                    os.path.join(ROOT, "oracle", "lco.c"), "-lm"], check=True)
    preload = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    code = f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import numpy as np
        from oracle import lco
        lco.LIB_PATH = {lib!r}
        from synth import gen, workloads as wls
        rs = np.random.default_rng(0)
        for agg, q in (("vote", 0), ("avg", 0), ("l1", 4), ("linf", 3)):
            for tie in ("parity", "zero"):
                wl = wls.Workload(name="san", tensors=[("a", 4096 + 640), ("b", 64), ("c", 130)],
                                  W=3, agg=agg, qbits=q, tie=tie, sync_names=("b",), sync_every=2,
                                  grad_dtype="bf16", theta_dtype="bf16")
                th, m, g = gen.host_theta(wl), gen.host_m(wl), gen.host_g(wl, 2)
                lco.step(wl, th, m, g, 2, debug=True)
                norms = {{"l1": lco.m1_all, "linf": lco.minf_all}}.get(agg, lambda *a: None)(wl, m, g)
                lco.step_range(wl, 64, 4096 + 64, norms, th[64:4096 + 64].copy(),
                               np.ascontiguousarray(m[:, 64:4096 + 64]),
                               np.ascontiguousarray(g[:, 64:4096 + 64]), 3, debug=True)
        x = rs.standard_normal((5, 4160)).astype(np.float32)
        x[:, ::7] = 0.0
        bits = lco.pack(x, 4100, 1)
        lco.vote(bits, 5, 4100, 1)
        sb, zb = lco.vote_bits(bits, 5, 4100, 2, lco.TIE_ZERO)
        wq = wls.Workload(name="q", tensors=[("a", 4096), ("b", 64)], W=5, agg="l1", qbits=4)
        codes, _ = lco.quant_l1(wq, x)
        lco.quant_linf(wq.with_(agg="linf"), x, 3)
        wire = lco.pack_codes(codes, 4100, 4)
        lco.unpack_sum(wire, 5, 4100, 4160, 4)
        wa = wls.flat("ap", 4100, W=5)
        lco.apply(wa, gen.host_theta(wa), gen.host_m(wa), gen.host_g(wa, 1), 1, sb, zb)
        lco.f32_to_bf16(x[0, :100]); lco.m1(x[0]); lco.minf(x[0])
        print("oracle clean")
    """
    r = _run_child(code, preload)
    assert r.returncode == 0 and "oracle clean" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


def test_host_library_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(OBJ, o) for o in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run __graft_entry__.build() first)")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    from communication_compressed_distributed_amd import build as libbuild
    lib = str(tmp_path / "liblioncub_san.so")
    host_objs = []
    for src in HOST_SRCS:
        host_obj = str(tmp_path / (src + ".san.o"))
        # sanitizer options on the host side only
        subprocess.run([hipcc, *libbuild.FLAGS, "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=undefined",
                        "-Xarch_host", "-fno-omit-frame-pointer", "-g",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                        "-c", "-o", host_obj, os.path.join(PKG, "csrc", src)], check=True)
        host_objs.append(host_obj)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-fPIC", "-shared",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-o", lib, *host_objs, *objs], check=True)
    rt = subprocess.run([hipcc.replace("bin/hipcc", "llvm/bin/clang"),
                         "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    code = f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import pytest
        import communication_compressed_distributed_amd._abi as abi
        abi.LIB_PATH = {lib!r}
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                              {os.path.join(ROOT, "tests", "test_abi_host.py")!r},
                              "-k", "not missing_library"]))
    """
    r = _run_child(code, rt)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
