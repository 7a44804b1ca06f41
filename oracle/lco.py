"""ctypes binding of the CPU oracle (liblco.so).

TEST INFRASTRUCTURE ONLY: for tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg.  Marshals NumPy arrays; all arithmetic is in lco.c.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblco.so")

VOTE, L1SUM, AVG, LINFSUM = 0, 1, 2, 3
TIE_PARITY, TIE_ZERO = 0, 1
M1_BLOCK = 4096


class Cfg(C.Structure):
    _fields_ = [
        ("d", C.c_int64), ("W", C.c_int32), ("n_tensors", C.c_int32),
        ("off", C.POINTER(C.c_int64)), ("sync_m", C.POINTER(C.c_uint8)),
        ("sync_every", C.c_int32), ("theta_bf16", C.c_int32), ("grad_bf16", C.c_int32),
        ("agg", C.c_int32), ("qbits", C.c_int32), ("tie_mode", C.c_int32),
        ("beta1", C.c_float), ("beta2", C.c_float), ("lr", C.c_float), ("wd", C.c_float),
        ("seed", C.c_uint64),
    ]


class Debug(C.Structure):
    _fields_ = [("bits", C.c_void_p), ("codes", C.c_void_p), ("counts", C.c_void_p),
                ("sums", C.c_void_p), ("sign", C.c_void_p), ("stats", C.c_void_p),
                ("mvar_max", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build
            build.build()
        L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.lco_bf16_to_f32.argtypes = [C.c_uint16]
        L.lco_bf16_to_f32.restype = C.c_float
        L.lco_f32_to_bf16.argtypes = [C.c_float]
        L.lco_f32_to_bf16.restype = C.c_uint16
        L.lco_bit.argtypes = [C.c_float, i64]
        L.lco_bit.restype = C.c_int
        L.lco_pack.argtypes = [i32, i64, i64, vp, i64, vp]
        L.lco_vote.argtypes = [i32, i64, i64, vp, i64, i32, vp, vp]
        L.lco_m1_block.argtypes = [vp, i64]
        L.lco_m1_block.restype = C.c_double
        L.lco_m1_finalize.argtypes = [vp, i64, i64]
        L.lco_m1_finalize.restype = C.c_double
        L.lco_m1.argtypes = [vp, i64]
        L.lco_m1.restype = C.c_double
        L.lco_q1.argtypes = [C.c_float, C.c_double, i32]
        L.lco_q1.restype = C.c_int8
        L.lco_quant_l1.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp]
        L.lco_c_row.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp]
        L.lco_m1_all.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp]
        L.lco_m1_partials.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp]
        L.lco_step_range.argtypes = [C.POINTER(Cfg), i64, i64, vp, vp, vp, vp, i64, i64,
                                     C.POINTER(Debug)]
        L.lco_step.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp, i64, C.POINTER(Debug)]
        L.lco_vote_bits.argtypes = [i32, i64, i64, vp, i64, i32, vp, vp]
        L.lco_apply.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp, i64, vp, vp]
        L.lco_pack_codes.argtypes = [i32, i64, i64, i32, vp, vp]
        L.lco_unpack_sum.argtypes = [i32, i64, i64, i32, vp, vp, vp]
        L.lco_unpack_sum_bits.argtypes = [i32, i64, i64, i32, vp, vp, vp]
        L.lco_splitmix64.argtypes = [C.c_uint64, C.c_uint64]
        L.lco_splitmix64.restype = C.c_uint64
        L.lco_minf.argtypes = [vp, i64]
        L.lco_minf.restype = C.c_double
        L.lco_sr_u32.argtypes = [C.c_uint64, i64, i32, i64, i32, i64]
        L.lco_sr_u32.restype = C.c_uint32
        L.lco_qinf.argtypes = [C.c_float, C.c_double, i32, C.c_uint32]
        L.lco_qinf.restype = C.c_int8
        L.lco_quant_linf.argtypes = [C.POINTER(Cfg), i64, vp, i64, vp, vp]
        L.lco_minf_all.argtypes = [C.POINTER(Cfg), i64, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class OracleCfg:
    """Holds a Cfg plus the arrays it points into (kept alive here)."""

    def __init__(self, wl, d=None, offsets=None):
        self.wl = wl
        off = np.asarray(offsets if offsets is not None else wl.offsets, dtype=np.int64)
        self.off = np.ascontiguousarray(off)
        flags = [1 if nm in wl.sync_names else 0 for nm, _ in wl.tensors]
        self.sync = np.asarray(flags, dtype=np.uint8) if any(flags) else None
        c = Cfg()
        c.d = int(d if d is not None else wl.d)
        c.W = wl.W
        c.n_tensors = len(self.off) - 1
        c.off = self.off.ctypes.data_as(C.POINTER(C.c_int64))
        c.sync_m = (self.sync.ctypes.data_as(C.POINTER(C.c_uint8)) if self.sync is not None
                    else C.POINTER(C.c_uint8)())
        c.sync_every = wl.sync_every
        c.theta_bf16 = 1 if wl.theta_dtype == "bf16" else 0
        c.grad_bf16 = 1 if wl.grad_dtype == "bf16" else 0
        c.agg = {"l1": L1SUM, "avg": AVG, "linf": LINFSUM}.get(wl.agg, VOTE)
        c.qbits = wl.qbits
        c.tie_mode = TIE_ZERO if wl.tie == "zero" else TIE_PARITY
        c.beta1, c.beta2, c.lr, c.wd = wl.beta1, wl.beta2, wl.lr, wl.wd
        c.seed = wl.sr_seed
        self.c = c

    @property
    def ref(self):
        return C.byref(self.c)


# ----------------------------------------------------------- functions ----

def f32_to_bf16(x):
    L = lib()
    return np.array([L.lco_f32_to_bf16(float(v)) for v in np.asarray(x, np.float32).ravel()],
                    dtype=np.uint16)


def bit(c, t):
    return lib().lco_bit(float(c), int(t))


def pack(x, d, t):
    """x[W][ld] fp32 -> bits[W][ld/64] uint64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    W, ld = x.shape
    bits = np.empty((W, ld // 64), dtype=np.uint64)
    lib().lco_pack(W, d, ld, _p(x), t, _p(bits))
    return bits


def vote(bits, W, d, t, tie_mode=TIE_PARITY):
    bits = np.ascontiguousarray(bits, dtype=np.uint64)
    ld = bits.shape[1] * 64
    counts = np.empty(d, dtype=np.uint8)
    sign = np.empty(d, dtype=np.int8)
    lib().lco_vote(W, d, ld, _p(bits), t, tie_mode, _p(counts), _p(sign))
    return counts, sign


def m1_block(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return lib().lco_m1_block(_p(a), a.size)


def m1_finalize(P, nT):
    P = np.ascontiguousarray(P, dtype=np.float64)
    return lib().lco_m1_finalize(_p(P), P.size, nT)


def m1(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return lib().lco_m1(_p(x), x.size)


def q1(c, m1v, qbits):
    return lib().lco_q1(float(c), float(m1v), int(qbits))


def quant_l1(wl, x):
    """x[W][ld] -> (codes[W][ld] int8 (zero past d), m1[W][n_tensors])."""
    cfg = OracleCfg(wl)
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    m1v = np.empty((wl.W, wl.n_tensors), dtype=np.float64)
    lib().lco_quant_l1(cfg.ref, x.shape[1], _p(x), _p(codes), _p(m1v))
    return codes, m1v


def splitmix64(seed, counter):
    return lib().lco_splitmix64(int(seed) & (2**64 - 1), int(counter) & (2**64 - 1))


def minf(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return lib().lco_minf(_p(x), x.size)


def sr_u32(seed, d, W, t, i, j):
    """The 32 random bits of element j of worker i at step t."""
    return lib().lco_sr_u32(int(seed) & (2**64 - 1), int(d), int(W), int(t), int(i), int(j))


def qinf(c, minf_v, qbits, r):
    """One max-norm stochastic code for the element's 32 random bits r."""
    return lib().lco_qinf(float(c), float(minf_v), int(qbits), int(r) & (2**32 - 1))


def quant_linf(wl, x, t):
    """Max-norm stochastic codes of x[W][ld] for step t -> (codes, minf[W][nT])."""
    cfg = OracleCfg(wl)
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    mv = np.empty((wl.W, wl.n_tensors), dtype=np.float64)
    lib().lco_quant_linf(cfg.ref, x.shape[1], _p(x), int(t), _p(codes), _p(mv))
    return codes, mv


def minf_all(wl, m, g):
    cfg = OracleCfg(wl)
    m = np.ascontiguousarray(m, dtype=np.float32)
    g = np.ascontiguousarray(g)
    out = np.empty((wl.W, wl.n_tensors), dtype=np.float64)
    lib().lco_minf_all(cfg.ref, m.shape[1], _p(m), _p(g), _p(out))
    return out


def c_row(wl, m_row, g_row):
    cfg = OracleCfg(wl)
    m_row = np.ascontiguousarray(m_row, dtype=np.float32)
    g_row = np.ascontiguousarray(g_row)
    out = np.empty(m_row.size, dtype=np.float32)
    lib().lco_c_row(cfg.ref, m_row.size, _p(m_row), _p(g_row), _p(out))
    return out


def m1_all(wl, m, g):
    cfg = OracleCfg(wl)
    m = np.ascontiguousarray(m, dtype=np.float32)
    g = np.ascontiguousarray(g)
    out = np.empty((wl.W, wl.n_tensors), dtype=np.float64)
    lib().lco_m1_all(cfg.ref, m.shape[1], _p(m), _p(g), _p(out))
    return out


def m1_partials(wl, m_row, g_row):
    """Block partials of a block-aligned run of one worker's row."""
    cfg = OracleCfg(wl)
    m_row = np.ascontiguousarray(m_row, dtype=np.float32)
    g_row = np.ascontiguousarray(g_row)
    out = np.empty((m_row.size + M1_BLOCK - 1) // M1_BLOCK, dtype=np.float64)
    lib().lco_m1_partials(cfg.ref, m_row.size, _p(m_row), _p(g_row), _p(out))
    return out


def _debug_arrays(wl, ncols, ldc, want):
    if not want:
        return None, None
    arr = {
        "bits": np.zeros((wl.W, ldc // 64), dtype=np.uint64) if ldc % 64 == 0 else None,
        "codes": np.zeros((wl.W, ldc), dtype=np.int8),
        "counts": np.zeros(ncols, dtype=np.uint8),
        "sums": np.zeros(ncols, dtype=np.int32),
        "sign": np.zeros(ncols, dtype=np.int8),
        "stats": np.zeros((wl.n_tensors, 4), dtype=np.uint64),
        "mvar_max": np.zeros(wl.n_tensors, dtype=np.float64),
    }
    dbg = Debug(*(None if arr[k] is None else arr[k].ctypes.data for k in
                  ("bits", "codes", "counts", "sums", "sign", "stats", "mvar_max")))
    return dbg, arr


def step(wl, theta, m, g, t, debug=False):
    """One whole step in place.  theta[d] (fp32 or uint16 bf16 bits),
    m[W][ld] fp32, g[W][ld] (fp32 or uint16 bf16 bits).  Returns the debug
    dict (bits, codes, counts, sums, sign) when debug=True."""
    cfg = OracleCfg(wl)
    for a in (theta, m, g):
        assert a.flags["C_CONTIGUOUS"]
    ld = m.shape[1]
    dbg, arr = _debug_arrays(wl, wl.d, ld, debug)
    lib().lco_step(cfg.ref, ld, _p(theta), _p(m), _p(g), t,
                   C.byref(dbg) if dbg is not None else None)
    return arr


def step_range(wl, j0, j1, m1v, theta_c, m_c, g_c, t, debug=False):
    """One step over columns [j0, j1) of chunk arrays (theta_c[j1-j0],
    m_c/g_c[W][ldc]); m1v[W][n_tensors] from the whole tensors (L1 path)."""
    cfg = OracleCfg(wl)
    ldc = m_c.shape[1]
    dbg, arr = _debug_arrays(wl, j1 - j0, ldc, debug)
    m1p = None if m1v is None else np.ascontiguousarray(m1v, dtype=np.float64)
    lib().lco_step_range(cfg.ref, j0, j1, _p(m1p), _p(theta_c), _p(m_c), _p(g_c), ldc, t,
                         C.byref(dbg) if dbg is not None else None)
    return arr


def vote_bits(bits, W, d, t, tie_mode=TIE_PARITY, zero=True):
    """-> (sign_bits[ld/64], zero_bits[ld/64] or None) uint64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint64)
    words = bits.shape[1]
    sb = np.empty(words, dtype=np.uint64)
    zb = np.empty(words, dtype=np.uint64) if zero else None
    lib().lco_vote_bits(W, d, words * 64, _p(bits), t, tie_mode, _p(sb), _p(zb))
    return sb, zb


def apply(wl, theta, m, g, t, sign_bits, zero_bits=None):
    """Steps 4-5 from a global sign given as bit planes, in place."""
    cfg = OracleCfg(wl)
    lib().lco_apply(cfg.ref, m.shape[1], _p(theta), _p(m), _p(g), t,
                    _p(np.ascontiguousarray(sign_bits, dtype=np.uint64)),
                    _p(None if zero_bits is None else np.ascontiguousarray(zero_bits, np.uint64)))


def pack_codes(codes, d, qbits):
    """codes[W][ld] int8 -> wire[W][(ld/32)*qbits] uint32."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    W, ld = codes.shape
    wire = np.empty((W, (ld // 32) * qbits), dtype=np.uint32)
    lib().lco_pack_codes(W, d, ld, qbits, _p(codes), _p(wire))
    return wire


def unpack_sum_bits(wire, W, d, ld, qbits, zero=True):
    """-> (sign_bits[ld/64], zero_bits[ld/64] or None) uint64 from the p-bit sums."""
    wire = np.ascontiguousarray(wire, dtype=np.uint32)
    sb = np.empty(ld // 64, dtype=np.uint64)
    zb = np.empty(ld // 64, dtype=np.uint64) if zero else None
    lib().lco_unpack_sum_bits(W, d, ld, qbits, _p(wire), _p(sb), _p(zb))
    return sb, zb


def unpack_sum(wire, W, d, ld, qbits):
    wire = np.ascontiguousarray(wire, dtype=np.uint32)
    sums = np.empty(d, dtype=np.int32)
    sign = np.empty(d, dtype=np.int8)
    lib().lco_unpack_sum(W, d, ld, qbits, _p(wire), _p(sums), _p(sign))
    return sums, sign
