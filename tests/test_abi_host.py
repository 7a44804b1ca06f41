"""Host-side checks of the C ABI (no GPU needed): the built library loads,
exports every entry point include/lioncub.h declares, sizes workspaces, and
rejects bad configurations and arguments before touching the device."""
import ctypes as C
import os
import re

import pytest

from communication_compressed_distributed_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "lioncub.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lioncub_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(_abi.EXPORTS)


def test_strerror_names_every_status():
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert _abi.lioncub_strerror(s) != "unknown status"
    assert _abi.lioncub_strerror(7) == "unknown status"


def test_step_static_rejects_before_device():
    """The allocation-free step checks its configuration, its pointers and
    the size of the fixed scratch array before any HIP call."""
    L = _abi.lib()
    p = C.c_void_p(4096)
    for bad in (dict(W=0), dict(ld=10000), dict(tensor_offsets=[0, 4000, 10000])):
        assert L.lioncub_step_static(C.byref(cfg(**bad)), None, p, p, p, 1) == _abi.EINVAL
    c = cfg()
    assert L.lioncub_step_static(None, None, p, p, p, 1) == _abi.EINVAL
    assert L.lioncub_step_static(C.byref(c), None, None, p, p, 1) == _abi.EINVAL
    assert L.lioncub_step_static(C.byref(c), None, p, p, p, 0) == _abi.EINVAL
    assert L.lioncub_step_static(C.byref(c), None, C.c_void_p(4100), p, p, 1) == _abi.EALIGN
    # the need is exactly lioncub_workspace_bytes: fits up to the array size
    big = cfg(d=350_000_000, ld=350_000_000, W=128, tensor_offsets=[0, 350_000_000])
    assert _abi.lioncub_workspace_bytes(big) > _abi.STATIC_SCRATCH_BYTES
    assert L.lioncub_step_static(C.byref(big), None, p, p, p, 1) == _abi.ESCRATCH
    assert "scratch" in _abi.lioncub_strerror(_abi.ESCRATCH)


def cfg(**kw):
    base = dict(d=10000, ld=10048, W=4, tensor_offsets=[0, 4096, 10000])
    base.update(kw)
    return _abi.make_config(**base)


def test_workspace_bytes_layout():
    # blocks: ceil(4096/4096) + ceil(5904/4096) = 3, one group of block
    # partials per tensor; 256-byte aligned pieces
    c = cfg()
    n = _abi.lioncub_workspace_bytes(c)
    blk = 3 * 16
    tens = 2 * 40
    grp = 2 * 16
    part = 4 * 3 * 8
    gval = 4 * 2 * 8
    m1 = 4 * 2 * 8
    bstat = 3 * 8 * 8
    gstat = 2 * 8 * 8
    al = lambda x: (x + 255) // 256 * 256
    assert n == (al(blk) + al(tens) + al(grp) + al(part) + al(gval) + 2 * al(m1) + al(bstat)
                 + al(gstat))
    big = cfg(d=1_313_626_112, ld=1_313_626_112, W=8,
              tensor_offsets=[0, 1_000_000_000 // 64 * 64, 1_313_626_112])
    assert _abi.lioncub_workspace_bytes(big) > 0


@pytest.mark.parametrize("bad", [
    dict(d=0, ld=64, tensor_offsets=[0, 0]),             # empty
    dict(ld=10000),                                       # ld not multiple of 64
    dict(ld=9984),                                        # ld < d
    dict(W=0), dict(W=256),                               # worker count
    dict(tensor_offsets=[0, 4000, 10000]),                # interior offset not % 64
    dict(tensor_offsets=[0, 4096, 9999]),                 # last offset != d
    dict(tensor_offsets=[0, 4096, 4096, 10000]),          # empty tensor
    dict(tensor_offsets=[64, 4096, 10000]),               # off[0] != 0
    dict(sync_every=0),
    dict(theta_dtype=2), dict(grad_dtype=-1),
    dict(agg=4), dict(agg=-1), dict(agg=_abi.AGG_L1SUM, qbits=1),
    dict(agg=_abi.AGG_L1SUM, qbits=9), dict(agg=_abi.AGG_LINFSUM, qbits=0),
    dict(agg=_abi.AGG_LINFSUM, qbits=9),
    dict(tie_mode=3),
    dict(lr=float("nan")), dict(beta1=float("inf")),
])
def test_invalid_config_rejected_before_device(bad):
    c = cfg(**bad)
    assert _abi.lioncub_workspace_bytes(c) == 0
    ctx = C.c_void_p()
    st = _abi.lib().lioncub_init(C.byref(ctx), C.byref(c), None, C.c_void_p(256), 1 << 30)
    assert st == _abi.EINVAL
    assert not ctx.value


@pytest.mark.parametrize("big", [
    dict(ld=2**40 + 64),                                          # row stride
    dict(d=2**40 + 64, ld=2**40 + 64, tensor_offsets=[0, 2**40 + 64]),
])
def test_unsupported_sizes_rejected_before_device(big):
    c = cfg(**big)
    assert _abi.lioncub_workspace_bytes(c) == 0
    ctx = C.c_void_p()
    st = _abi.lib().lioncub_init(C.byref(ctx), C.byref(c), None, C.c_void_p(256), 1 << 30)
    assert st == _abi.EUNSUPPORTED
    assert not ctx.value
    ok = cfg(d=2**40, ld=2**40, tensor_offsets=[0, 2**40])
    assert _abi.lioncub_workspace_bytes(ok) > 0


def test_workspace_checked_before_device():
    c = cfg()
    n = _abi.lioncub_workspace_bytes(c)
    L = _abi.lib()
    ctx = C.c_void_p()
    assert L.lioncub_init(C.byref(ctx), C.byref(c), None, None, n) == _abi.EWORKSPACE
    assert L.lioncub_init(C.byref(ctx), C.byref(c), None, C.c_void_p(256), n - 1) == _abi.EWORKSPACE
    assert L.lioncub_init(C.byref(ctx), C.byref(c), None, C.c_void_p(128), n) == _abi.EWORKSPACE
    assert L.lioncub_init(None, C.byref(c), None, C.c_void_p(256), n) == _abi.EINVAL


def test_null_context_and_arguments_rejected():
    L = _abi.lib()
    p = C.c_void_p(4096)
    assert L.lioncub_step(None, p, p, p, 1, None) == _abi.EINVAL
    assert L.lioncub_pack(None, p, 1, p) == _abi.EINVAL
    assert L.lioncub_vote(None, p, 1, p, p) == _abi.EINVAL
    assert L.lioncub_quant_l1(None, p, p, None) == _abi.EINVAL
    assert L.lioncub_unpack_sum(None, p, p, p) == _abi.EINVAL
    assert L.lioncub_unpack_sum_bits(None, p, p, None) == _abi.EINVAL
    assert L.lioncub_set_stream(None, None) == _abi.EINVAL
    assert L.lioncub_profile_begin(None, 4) == _abi.EINVAL
    assert L.lioncub_destroy(None) == _abi.OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library the product path raises."""
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "liblioncub.so"))
    with pytest.raises(ImportError):
        _abi.lib()
    with pytest.raises(ImportError):
        _abi.lioncub_workspace_bytes(cfg())
