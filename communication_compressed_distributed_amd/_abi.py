"""ctypes binding of liblioncub.so (include/lioncub.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of the library.  Device buffers are torch tensors on a ROCm device;
their data pointers and torch's current HIP stream are handed to the library.
Loading fails loudly (ImportError) when the built library is absent: there is
no fallback path.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblioncub.so")

OK, EINVAL, EALIGN, EWORKSPACE, EDEVICE, EUNSUPPORTED, ENOMEM, ESCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7)
STATIC_SCRATCH_BYTES = 64 << 20   # LIONCUB_STATIC_SCRATCH_BYTES
F32, BF16 = 0, 1
AGG_VOTE, AGG_L1SUM, AGG_AVG, AGG_LINFSUM = 0, 1, 2, 3
TIE_PARITY, TIE_ZERO = 0, 1
(K_VOTE_STEP, K_M1_PARTIAL, K_M1_FINALIZE, K_L1_STEP, K_PACK, K_VOTE, K_QUANT, K_VOTE_BITS,
 K_APPLY, K_PACK_CODES, K_UNPACK_SUM, K_AVG_STEP, K_STATS, K_LINF_STEP, K_QUANT_LINF,
 K_UNPACK_BITS, K_COUNT) = range(17)
KERNEL_NAMES = ["vote_step", "m1_partial", "m1_finalize", "l1_step", "pack", "vote", "quant",
                "vote_bits", "apply", "pack_codes", "unpack_sum", "avg_step", "stats",
                "linf_step", "quant_linf", "unpack_bits"]

EXPORTS = ["lioncub_workspace_bytes", "lioncub_init", "lioncub_set_stream", "lioncub_step",
           "lioncub_step_static",
           "lioncub_pack", "lioncub_vote", "lioncub_quant_l1", "lioncub_quant_linf",
           "lioncub_vote_bits",
           "lioncub_apply", "lioncub_pack_codes", "lioncub_unpack_sum", "lioncub_unpack_sum_bits",
           "lioncub_profile_begin",
           "lioncub_profile_end", "lioncub_destroy", "lioncub_strerror"]


class lioncub_config(C.Structure):
    _fields_ = [
        ("d", C.c_int64), ("ld", C.c_int64), ("W", C.c_int32), ("n_tensors", C.c_int32),
        ("tensor_offsets", C.POINTER(C.c_int64)), ("sync_m", C.POINTER(C.c_uint8)),
        ("sync_every", C.c_int32), ("theta_dtype", C.c_int32), ("grad_dtype", C.c_int32),
        ("agg", C.c_int32), ("qbits", C.c_int32), ("tie_mode", C.c_int32),
        ("beta1", C.c_float), ("beta2", C.c_float), ("lr", C.c_float), ("wd", C.c_float),
        ("sr_seed", C.c_uint64),
    ]


class lioncub_debug(C.Structure):
    _fields_ = [("bits", C.c_void_p), ("codes", C.c_void_p), ("counts", C.c_void_p),
                ("sums", C.c_void_p), ("sign", C.c_void_p), ("m1", C.c_void_p),
                ("stats", C.c_void_p), ("mvar_max", C.c_void_p)]


_lib = None


def lib():
    """Load liblioncub.so (built by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        cfgp = C.POINTER(lioncub_config)
        L.lioncub_workspace_bytes.argtypes = [cfgp]
        L.lioncub_workspace_bytes.restype = C.c_size_t
        L.lioncub_init.argtypes = [C.POINTER(vp), cfgp, vp, vp, C.c_size_t]
        L.lioncub_init.restype = C.c_int
        L.lioncub_set_stream.argtypes = [vp, vp]
        L.lioncub_set_stream.restype = C.c_int
        L.lioncub_step.argtypes = [vp, vp, vp, vp, i64, C.POINTER(lioncub_debug)]
        L.lioncub_step.restype = C.c_int
        L.lioncub_step_static.argtypes = [cfgp, vp, vp, vp, vp, i64]
        L.lioncub_step_static.restype = C.c_int
        L.lioncub_pack.argtypes = [vp, vp, i64, vp]
        L.lioncub_pack.restype = C.c_int
        L.lioncub_vote.argtypes = [vp, vp, i64, vp, vp]
        L.lioncub_vote.restype = C.c_int
        L.lioncub_quant_l1.argtypes = [vp, vp, vp, vp]
        L.lioncub_quant_l1.restype = C.c_int
        L.lioncub_quant_linf.argtypes = [vp, vp, C.c_int64, vp, vp]
        L.lioncub_quant_linf.restype = C.c_int
        L.lioncub_vote_bits.argtypes = [vp, vp, i64, vp, vp]
        L.lioncub_vote_bits.restype = C.c_int
        L.lioncub_apply.argtypes = [vp, vp, vp, vp, i64, vp, vp]
        L.lioncub_apply.restype = C.c_int
        L.lioncub_pack_codes.argtypes = [vp, vp, vp]
        L.lioncub_pack_codes.restype = C.c_int
        L.lioncub_unpack_sum.argtypes = [vp, vp, vp, vp]
        L.lioncub_unpack_sum.restype = C.c_int
        L.lioncub_unpack_sum_bits.argtypes = [vp, vp, vp, vp]
        L.lioncub_unpack_sum_bits.restype = C.c_int
        L.lioncub_profile_begin.argtypes = [vp, i32]
        L.lioncub_profile_begin.restype = C.c_int
        L.lioncub_profile_end.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
        L.lioncub_profile_end.restype = C.c_int
        L.lioncub_destroy.argtypes = [vp]
        L.lioncub_destroy.restype = C.c_int
        L.lioncub_strerror.argtypes = [C.c_int]
        L.lioncub_strerror.restype = C.c_char_p
        _lib = L
    return _lib


class LionCubError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().lioncub_strerror(status).decode()
        super().__init__(f"{fn} failed: {status} ({msg})")
        self.status = status


def _check(fn, status):
    if status != OK:
        raise LionCubError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def make_config(d, ld, W, tensor_offsets, sync_m=None, sync_every=1, theta_dtype=F32,
                grad_dtype=F32, agg=AGG_VOTE, qbits=0, tie_mode=TIE_PARITY, beta1=0.9,
                beta2=0.99, lr=1e-4, wd=0.1, sr_seed=0):
    """A lioncub_config plus the host arrays it points to (kept alive on it)."""
    cfg = lioncub_config()
    offs = (C.c_int64 * len(tensor_offsets))(*[int(v) for v in tensor_offsets])
    cfg.d, cfg.ld, cfg.W, cfg.n_tensors = int(d), int(ld), int(W), len(tensor_offsets) - 1
    cfg.tensor_offsets = C.cast(offs, C.POINTER(C.c_int64))
    cfg._offs = offs
    if sync_m is not None:
        flags = (C.c_uint8 * len(sync_m))(*[1 if f else 0 for f in sync_m])
        cfg.sync_m = C.cast(flags, C.POINTER(C.c_uint8))
        cfg._flags = flags
    cfg.sync_every, cfg.theta_dtype, cfg.grad_dtype = sync_every, theta_dtype, grad_dtype
    cfg.agg, cfg.qbits, cfg.tie_mode = agg, qbits, tie_mode
    cfg.beta1, cfg.beta2, cfg.lr, cfg.wd = beta1, beta2, lr, wd
    cfg.sr_seed = int(sr_seed) & (2**64 - 1)
    return cfg


# ------------------------------------------------ the C ABI, same names ----

def lioncub_workspace_bytes(cfg):
    return lib().lioncub_workspace_bytes(C.byref(cfg))


def lioncub_init(cfg, stream, workspace):
    """-> ctx handle (c_void_p).  workspace: torch uint8 device tensor."""
    ctx = C.c_void_p()
    _check("lioncub_init", lib().lioncub_init(C.byref(ctx), C.byref(cfg), stream,
                                              _ptr(workspace), workspace.numel()))
    return ctx


def lioncub_set_stream(ctx, stream):
    _check("lioncub_set_stream", lib().lioncub_set_stream(ctx, stream))


def lioncub_step(ctx, theta, m, g, t, dbg=None):
    d = None
    if dbg is not None:
        d = lioncub_debug(*(None if dbg.get(k) is None else dbg[k].data_ptr()
                            for k in ("bits", "codes", "counts", "sums", "sign", "m1",
                                      "stats", "mvar_max")))
    _check("lioncub_step", lib().lioncub_step(ctx, _ptr(theta), _ptr(m), _ptr(g), int(t),
                                              C.byref(d) if d is not None else None))


def lioncub_step_static(cfg, stream, theta, m, g, t):
    """The allocation-free step: no context, no workspace (the library's
    fixed scratch array); `stream` is a HIP stream handle (c_void_p)."""
    _check("lioncub_step_static", lib().lioncub_step_static(C.byref(cfg), stream, _ptr(theta),
                                                            _ptr(m), _ptr(g), int(t)))


def lioncub_pack(ctx, x, t, bits):
    _check("lioncub_pack", lib().lioncub_pack(ctx, _ptr(x), int(t), _ptr(bits)))


def lioncub_vote(ctx, bits, t, counts=None, sign=None):
    _check("lioncub_vote", lib().lioncub_vote(ctx, _ptr(bits), int(t), _ptr(counts), _ptr(sign)))


def lioncub_quant_l1(ctx, x, codes, m1=None):
    _check("lioncub_quant_l1", lib().lioncub_quant_l1(ctx, _ptr(x), _ptr(codes), _ptr(m1)))


def lioncub_quant_linf(ctx, x, t, codes, minf=None):
    _check("lioncub_quant_linf",
           lib().lioncub_quant_linf(ctx, _ptr(x), int(t), _ptr(codes), _ptr(minf)))


def lioncub_vote_bits(ctx, bits, t, sign_bits, zero_bits=None):
    _check("lioncub_vote_bits", lib().lioncub_vote_bits(ctx, _ptr(bits), int(t), _ptr(sign_bits),
                                                        _ptr(zero_bits)))


def lioncub_apply(ctx, theta, m, g, t, sign_bits, zero_bits=None):
    _check("lioncub_apply", lib().lioncub_apply(ctx, _ptr(theta), _ptr(m), _ptr(g), int(t),
                                                _ptr(sign_bits), _ptr(zero_bits)))


def lioncub_pack_codes(ctx, codes, wire):
    _check("lioncub_pack_codes", lib().lioncub_pack_codes(ctx, _ptr(codes), _ptr(wire)))


def lioncub_unpack_sum(ctx, wire, sums=None, sign=None):
    _check("lioncub_unpack_sum", lib().lioncub_unpack_sum(ctx, _ptr(wire), _ptr(sums), _ptr(sign)))


def lioncub_unpack_sum_bits(ctx, wire, sign_bits, zero_bits=None):
    _check("lioncub_unpack_sum_bits",
           lib().lioncub_unpack_sum_bits(ctx, _ptr(wire), _ptr(sign_bits), _ptr(zero_bits)))


def lioncub_profile_begin(ctx, capacity):
    _check("lioncub_profile_begin", lib().lioncub_profile_begin(ctx, int(capacity)))


def lioncub_profile_end(ctx):
    """-> {kernel name: (total ms, launches)}"""
    ms = (C.c_double * K_COUNT)()
    n = (C.c_int32 * K_COUNT)()
    _check("lioncub_profile_end", lib().lioncub_profile_end(ctx, ms, n))
    return {KERNEL_NAMES[k]: (ms[k], n[k]) for k in range(K_COUNT)}


def lioncub_destroy(ctx):
    _check("lioncub_destroy", lib().lioncub_destroy(ctx))


def lioncub_strerror(status):
    return lib().lioncub_strerror(int(status)).decode()
