"""Host-side argument checks for the LionCub wrapper.

The C ABI takes plain device pointers and cannot see how large a buffer is,
so a tensor that is too small, strided or of the wrong element type would be
read or written out of bounds by a kernel.  Every tensor the wrapper passes
is checked here first: device, contiguity, element type and extent (at
least the elements the call touches, as laid out in include/lioncub.h).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Spec:
    d: int
    ld: int
    W: int
    n_tensors: int
    theta_dtype: str   # "f32" | "bf16"
    grad_dtype: str
    qbits: int


def _dt():
    import torch
    return {"f32": (torch.float32,), "bf16": (torch.bfloat16,), "f64": (torch.float64,),
            "u64": (torch.int64, torch.uint64), "u32": (torch.int32, torch.uint32),
            "i32": (torch.int32,), "i8": (torch.int8,), "u8": (torch.uint8,)}


def need(name, t, device, kind, numel, optional=False):
    """Raise ValueError unless t is a contiguous tensor of one of the dtypes
    of `kind` on `device` holding at least `numel` elements."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: required")
    dts = _dt()[kind]
    if t.dtype not in dts:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dts))}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the context is on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call touches {numel}")


def state(s, dev, theta, m, g):
    need("theta", theta, dev, s.theta_dtype, s.d)
    need("m", m, dev, "f32", s.W * s.ld)
    need("g", g, dev, s.grad_dtype, s.W * s.ld)


def step(s, dev, theta, m, g, debug):
    state(s, dev, theta, m, g)
    if debug is None:
        return
    unknown = set(debug) - {"bits", "codes", "counts", "sums", "sign", "m1", "stats", "mvar_max"}
    if unknown:
        raise ValueError(f"debug: unknown outputs {sorted(unknown)}")
    g_ = debug.get
    need("debug.bits", g_("bits"), dev, "u64", s.W * (s.ld // 64), optional=True)
    need("debug.codes", g_("codes"), dev, "i8", s.W * s.ld, optional=True)
    need("debug.counts", g_("counts"), dev, "u8", s.d, optional=True)
    need("debug.sums", g_("sums"), dev, "i32", s.d, optional=True)
    need("debug.sign", g_("sign"), dev, "i8", s.d, optional=True)
    need("debug.m1", g_("m1"), dev, "f64", s.W * s.n_tensors, optional=True)
    need("debug.stats", g_("stats"), dev, "u64", 4 * s.n_tensors, optional=True)
    need("debug.mvar_max", g_("mvar_max"), dev, "f64", s.n_tensors, optional=True)


def pack(s, dev, x, bits):
    need("x", x, dev, "f32", s.W * s.ld)
    need("bits", bits, dev, "u64", s.W * (s.ld // 64))


def vote(s, dev, bits, counts, sign):
    need("bits", bits, dev, "u64", s.W * (s.ld // 64))
    need("counts", counts, dev, "u8", s.d, optional=True)
    need("sign", sign, dev, "i8", s.d, optional=True)


def quant(s, dev, x, codes, norm):
    need("x", x, dev, "f32", s.W * s.ld)
    need("codes", codes, dev, "i8", s.W * s.ld)
    need("norm", norm, dev, "f64", s.W * s.n_tensors, optional=True)


def vote_bits(s, dev, bits, sign_bits, zero_bits):
    need("bits", bits, dev, "u64", s.W * (s.ld // 64))
    need("sign_bits", sign_bits, dev, "u64", s.ld // 64)
    need("zero_bits", zero_bits, dev, "u64", s.ld // 64, optional=True)


def apply(s, dev, theta, m, g, sign_bits, zero_bits):
    state(s, dev, theta, m, g)
    need("sign_bits", sign_bits, dev, "u64", s.ld // 64)
    need("zero_bits", zero_bits, dev, "u64", s.ld // 64, optional=True)


def pack_codes(s, dev, codes, wire):
    need("codes", codes, dev, "i8", s.W * s.ld)
    need("wire", wire, dev, "u32", s.W * (s.ld // 32) * max(s.qbits, 0))


def unpack_sum(s, dev, wire, sums, sign):
    need("wire", wire, dev, "u32", s.W * (s.ld // 32) * max(s.qbits, 0))
    need("sums", sums, dev, "i32", s.d, optional=True)
    need("sign", sign, dev, "i8", s.d, optional=True)


def unpack_sum_bits(s, dev, wire, sign_bits, zero_bits):
    need("wire", wire, dev, "u32", s.W * (s.ld // 32) * max(s.qbits, 0))
    need("sign_bits", sign_bits, dev, "u64", s.ld // 64)
    need("zero_bits", zero_bits, dev, "u64", s.ld // 64, optional=True)
