"""ctypes binding of the measurement library liblioncub_probe.so
(include/lioncub_probe.h), same names as its C ABI.

Measurement only, beside the step library: STREAM-style reference kernels
and a trivial-arithmetic probe of the fused step's access pattern, used by
the benchmark to report ceilings next to the published peak.  Argument
marshalling only; raises ImportError when the library is not built.
"""
import ctypes as C
import os

from ._abi import LionCubError, _ptr

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblioncub_probe.so")

PROBE_READ, PROBE_COPY, PROBE_TRIAD = 0, 1, 2
PROBE_CACHED, PROBE_MASKED = 1, 2     # lioncub_probe_step_pattern flags
EXPORTS = ["lioncub_probe_stream", "lioncub_probe_step_pattern", "lioncub_probe_panel_pattern"]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.lioncub_probe_stream.argtypes = [i32, vp, vp, vp, i64, vp]
        L.lioncub_probe_stream.restype = C.c_int
        L.lioncub_probe_step_pattern.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, C.c_float,
                                                 C.c_float, i32, vp]
        L.lioncub_probe_step_pattern.restype = C.c_int
        L.lioncub_probe_panel_pattern.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, C.c_float,
                                                  C.c_float, i32, vp]
        L.lioncub_probe_panel_pattern.restype = C.c_int
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise LionCubError(fn, status)


def lioncub_probe_stream(kind, a, b, c, n, stream):
    _check("lioncub_probe_stream",
           lib().lioncub_probe_stream(int(kind), _ptr(a), _ptr(b), _ptr(c), int(n), stream))


def lioncub_probe_step_pattern(theta, m, g, d, ld, W, theta_dtype, grad_dtype, beta2, lr, stream,
                               flags=0):
    _check("lioncub_probe_step_pattern",
           lib().lioncub_probe_step_pattern(_ptr(theta), _ptr(m), _ptr(g), int(d), int(ld),
                                            int(W), int(theta_dtype), int(grad_dtype),
                                            float(beta2), float(lr), int(flags), stream))


def lioncub_probe_panel_pattern(theta, m, g, d, ld, W, theta_dtype, grad_dtype, beta2, lr,
                                panel_blocks, stream):
    _check("lioncub_probe_panel_pattern",
           lib().lioncub_probe_panel_pattern(_ptr(theta), _ptr(m), _ptr(g), int(d), int(ld),
                                             int(W), int(theta_dtype), int(grad_dtype),
                                             float(beta2), float(lr), int(panel_blocks), stream))
