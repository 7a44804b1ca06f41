"""Host-side checks of the measurement library liblioncub_probe.so (no GPU):
it loads, exports exactly what include/lioncub_probe.h declares, and rejects
bad arguments before touching the device.  The step library no longer
exports any measurement kernel."""
import ctypes as C
import os
import re

from communication_compressed_distributed_amd import _abi, _probe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_probe_library_exports_its_header():
    txt = open(os.path.join(ROOT, "include", "lioncub_probe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = sorted(set(re.findall(r"\b(lioncub_probe_[a-z0-9_]+)\s*\(", txt)))
    assert names == sorted(_probe.EXPORTS)
    L = _probe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert not hasattr(_abi.lib(), "lioncub_stream_probe")


def test_probe_stream_rejects_bad_arguments_before_device():
    L = _probe.lib()
    p = C.c_void_p(256)
    assert L.lioncub_probe_stream(3, p, p, p, 4096, None) == _abi.EINVAL        # kind
    assert L.lioncub_probe_stream(0, p, p, p, 4095, None) == _abi.EINVAL        # n % 4096
    assert L.lioncub_probe_stream(0, p, p, p, 0, None) == _abi.EINVAL
    assert L.lioncub_probe_stream(2, p, None, p, 4096, None) == _abi.EINVAL     # triad needs b
    assert L.lioncub_probe_stream(1, C.c_void_p(260), p, p, 4096, None) == _abi.EALIGN


def test_probe_pattern_rejects_bad_arguments_before_device():
    L = _probe.lib()
    p = C.c_void_p(256)
    ok = dict(d=5000, ld=5056, W=4, td=0, gd=0, flags=0)

    def call(theta=p, m=p, g=p, **kw):
        a = dict(ok, **kw)
        return L.lioncub_probe_step_pattern(theta, m, g, a["d"], a["ld"], a["W"], a["td"], a["gd"],
                                            0.99, 1e-4, a["flags"], None)
    assert call(flags=64) == _abi.EINVAL                 # unknown bit
    assert call(flags=1 | 4) == _abi.EINVAL              # cap with plain accesses
    assert call(flags=2 | 16) == _abi.EINVAL             # drain with the masked path
    assert call(flags=4 | 16) == _abi.EINVAL             # cap and drain together
    assert call(theta=None) == _abi.EINVAL
    assert call(d=0) == _abi.EINVAL
    assert call(ld=5000) == _abi.EINVAL                  # not a multiple of 64
    assert call(ld=4992) == _abi.EINVAL                  # < d
    assert call(W=0) == _abi.EINVAL and call(W=256) == _abi.EINVAL
    assert call(td=2) == _abi.EINVAL and call(gd=-1) == _abi.EINVAL
    assert call(m=C.c_void_p(264)) == _abi.EALIGN
