"""Host-side argument checks of the LionCub wrapper (no GPU needed): every
tensor is checked for element type, contiguity, device and extent before its
pointer reaches the C ABI."""
import pytest
import torch

from communication_compressed_distributed_amd import _checks

CPU = torch.device("cpu")
S = _checks.Spec(d=1000, ld=1024, W=3, n_tensors=2, theta_dtype="bf16", grad_dtype="f32",
                 qbits=4)


def good_state():
    return (torch.zeros(1000, dtype=torch.bfloat16), torch.zeros((3, 1024)),
            torch.zeros((3, 1024)))


def test_good_arguments_pass():
    th, m, g = good_state()
    _checks.step(S, CPU, th, m, g, None)
    _checks.step(S, CPU, th, m, g, {
        "bits": torch.zeros((3, 16), dtype=torch.int64), "codes": torch.zeros((3, 1024), dtype=torch.int8),
        "counts": torch.zeros(1000, dtype=torch.uint8), "sums": torch.zeros(1000, dtype=torch.int32),
        "sign": torch.zeros(1000, dtype=torch.int8), "m1": torch.zeros((3, 2), dtype=torch.float64),
        "stats": torch.zeros((2, 4), dtype=torch.int64), "mvar_max": torch.zeros(2, dtype=torch.float64)})
    _checks.pack(S, CPU, m, torch.zeros((3, 16), dtype=torch.int64))
    _checks.vote(S, CPU, torch.zeros((3, 16), dtype=torch.int64), None, torch.zeros(1000, dtype=torch.int8))
    _checks.quant(S, CPU, m, torch.zeros((3, 1024), dtype=torch.int8), None)
    _checks.vote_bits(S, CPU, torch.zeros((3, 16), dtype=torch.int64), torch.zeros(16, dtype=torch.int64), None)
    _checks.apply(S, CPU, th, m, g, torch.zeros(16, dtype=torch.int64), torch.zeros(16, dtype=torch.int64))
    _checks.pack_codes(S, CPU, torch.zeros((3, 1024), dtype=torch.int8), torch.zeros((3, 128), dtype=torch.int32))
    _checks.unpack_sum(S, CPU, torch.zeros((3, 128), dtype=torch.int32), torch.zeros(1000, dtype=torch.int32), None)
    _checks.unpack_sum_bits(S, CPU, torch.zeros((3, 128), dtype=torch.int32), torch.zeros(16, dtype=torch.int64), None)


@pytest.mark.parametrize("case", [
    "theta short", "theta f32", "m short", "m strided", "m f64", "g bf16", "debug codes short",
    "debug bits i32", "debug unknown", "stats short", "wire short", "sign u8", "bits missing",
    "planes short", "planes i32"])
def test_bad_arguments_raise(case):
    th, m, g = good_state()
    with pytest.raises(ValueError):
        if case == "theta short":
            _checks.step(S, CPU, th[1:], m, g, None)
        elif case == "theta f32":
            _checks.step(S, CPU, th.float(), m, g, None)
        elif case == "m short":
            _checks.step(S, CPU, th, m[:2], g, None)
        elif case == "m strided":
            _checks.step(S, CPU, th, torch.zeros((3, 2048))[:, ::2], g, None)
        elif case == "m f64":
            _checks.step(S, CPU, th, m.double(), g, None)
        elif case == "g bf16":
            _checks.step(S, CPU, th, m, g.bfloat16(), None)
        elif case == "debug codes short":
            _checks.step(S, CPU, th, m, g, {"codes": torch.zeros((3, 1000), dtype=torch.int8)})
        elif case == "debug bits i32":
            _checks.step(S, CPU, th, m, g, {"bits": torch.zeros((3, 32), dtype=torch.int32)})
        elif case == "debug unknown":
            _checks.step(S, CPU, th, m, g, {"count": torch.zeros(1000, dtype=torch.uint8)})
        elif case == "stats short":
            _checks.step(S, CPU, th, m, g, {"stats": torch.zeros(4, dtype=torch.int64)})
        elif case == "wire short":
            _checks.pack_codes(S, CPU, torch.zeros((3, 1024), dtype=torch.int8),
                               torch.zeros((3, 127), dtype=torch.int32))
        elif case == "sign u8":
            _checks.vote(S, CPU, torch.zeros((3, 16), dtype=torch.int64), None,
                         torch.zeros(1000, dtype=torch.uint8))
        elif case == "bits missing":
            _checks.vote_bits(S, CPU, torch.zeros((3, 16), dtype=torch.int64), None, None)
        elif case == "planes short":
            _checks.unpack_sum_bits(S, CPU, torch.zeros((3, 128), dtype=torch.int32),
                                    torch.zeros(15, dtype=torch.int64), None)
        elif case == "planes i32":
            _checks.unpack_sum_bits(S, CPU, torch.zeros((3, 128), dtype=torch.int32),
                                    torch.zeros(16, dtype=torch.int64), torch.zeros(32, dtype=torch.int32))


def test_device_must_match():
    th, m, g = good_state()
    with pytest.raises(ValueError):
        _checks.step(S, torch.device("cuda", 0), th, m, g, None)


@pytest.mark.parametrize("kw", [dict(theta_dtype="fp16"), dict(grad_dtype="f16"),
                                dict(tie="even"), dict(agg="sum")])
def test_lioncub_rejects_unknown_names_before_allocating(kw):
    from communication_compressed_distributed_amd import LionCub
    with pytest.raises(ValueError):
        LionCub(d=4096, W=2, device="cpu", **kw)


def test_static_step_wrapper_checks_before_the_library(monkeypatch):
    """StaticStep validates its options and the scratch-array size at
    construction and every tensor before the allocation-free entry point is
    called (here the entry point is replaced: nothing reaches a device)."""
    import communication_compressed_distributed_amd as lc
    from communication_compressed_distributed_amd import _abi

    with pytest.raises(ValueError):
        lc.StaticStep(d=1000, W=3, agg="sum")
    with pytest.raises(lc.LionCubError) as e:
        lc.StaticStep(d=350_000_000, W=128, agg="l1", qbits=4)
    assert e.value.status == _abi.ESCRATCH
    st = lc.StaticStep(d=1000, W=3, tensor_offsets=[0, 512, 1000], theta_dtype="bf16", agg="l1",
                       qbits=4)
    assert st.ld == 1024 and st.n_tensors == 2
    calls = []
    monkeypatch.setattr(lc, "lioncub_step_static", lambda *a: calls.append(a))
    monkeypatch.setattr(lc._abi, "_stream_handle", lambda s=None: None)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda dev=None: None)
    th, m, g = good_state()
    st.step(th, m, g, 1)
    assert len(calls) == 1 and calls[0][5] == 1
    with pytest.raises(ValueError):
        st.step(th[:999], m, g, 2)
    with pytest.raises(ValueError):
        st.step(th, m.t(), g, 2)
    assert len(calls) == 1
