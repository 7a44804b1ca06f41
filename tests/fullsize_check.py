"""Every-element comparison of one full-size device step with the CPU oracle.

The device state before the step is snapshotted on the device (the 288 GB of
HBM hold the largest workload's state twice), the step runs with the
production kernels, and then block-aligned column chunks of the snapshot,
the gradients and the result are copied to pinned host buffers and checked:

1. on the quantised paths, the oracle's norm of every (worker, tensor) pair,
   its block partials computed chunk by chunk in the fixed block order and
   then finalised, against the library's, bit for bit;
2. the oracle's serial step (lco_step_range) on every column of every
   chunk, run by P host threads on disjoint column ranges (a column's result
   depends on nothing outside it once the norms are known), against the
   device's theta and m, within the fp32 / bf16 bar and then bit for bit.

Test infrastructure: calls the oracle and the library, holds no arithmetic
of the method itself.
"""
import ctypes as C
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import lco
from tests.harness import check_float_state

BLOCK = lco.M1_BLOCK


def _say(*a):
    print("[every-element]", *a, flush=True)


def column_chunks(wl, target):
    """Cut [0, d) into chunks of about `target` columns whose every cut lies
    on a block boundary of the tensor it falls in: whole small tensors are
    grouped, a large tensor is cut at its own start + k * target (target a
    multiple of the block).  Returns [(j0, j1, [(T, a, b), ...])] with the
    tensor pieces [a, b) each chunk holds."""
    assert target % BLOCK == 0
    off = wl.offsets
    chunks, cur, j0 = [], [], 0
    for T in range(wl.n_tensors):
        a, b = off[T], off[T + 1]
        s = a
        while s < b:
            e = min(b, s + target)
            if cur and (e - j0) > target:
                chunks.append((j0, s, cur))
                cur, j0 = [], s
            cur.append((T, s, e))
            s = e
    if cur:
        chunks.append((j0, wl.d, cur))
    return chunks


class Pinned:
    """Reusable pinned host buffers, one per name."""

    def __init__(self):
        self.buf = {}

    def get(self, name, shape, dtype):
        import torch
        n = int(np.prod(shape))
        b = self.buf.get(name)
        if b is None or b.numel() < n or b.dtype != dtype:
            b = torch.empty(n, dtype=dtype, pin_memory=True)
            self.buf[name] = b
        return b[:n].view(*shape)


def _host_rows(pin, name, x, j0, j1):
    """x[:, j0:j1] (device [W][ld]) into a pinned [W][j1-j0] buffer, row by
    row (contiguous device reads); returns a NumPy view (bf16 as uint16)."""
    import torch
    W = x.shape[0]
    dt = torch.int16 if x.dtype == torch.bfloat16 else x.dtype
    h = pin.get(name, (W, j1 - j0), dt)
    src = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    for i in range(W):
        h[i].copy_(src[i, j0:j1], non_blocking=True)
    return h


def _host_vec(pin, name, x, j0, j1):
    import torch
    dt = torch.int16 if x.dtype == torch.bfloat16 else x.dtype
    h = pin.get(name, (j1 - j0,), dt)
    src = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
    h.copy_(src[j0:j1], non_blocking=True)
    return h


def _np(t, bf16=False):
    a = t.numpy()
    return a.view(np.uint16) if bf16 else a


def _check(pool, name, got, want, bf16):
    """Bit equality row by row on the pool's threads; on any difference the
    full bar (tolerance first, then bits) reports what differs."""
    u = np.uint16 if bf16 else np.uint32
    same = list(pool.map(lambda i: np.array_equal(got[i].view(u), want[i].view(u)),
                         range(got.shape[0])))
    if not all(same):
        check_float_state(name, got, want, bf16=bf16)
        raise AssertionError(f"{name}: bit patterns differ")


def oracle_norms(wl, m0, g, pin, pool, chunks):
    """The oracle's M1 (L1 path) or max |c| (max-norm path) of every
    (worker, tensor) pair from the device arrays m0, g, streamed in chunks."""
    import torch
    L = lco.lib()
    cfg = lco.OracleCfg(wl)
    W, off = wl.W, wl.offsets
    gb = wl.grad_dtype == "bf16"
    nblk = [(off[T + 1] - off[T] + BLOCK - 1) // BLOCK for T in range(wl.n_tensors)]
    parts = [[np.empty(nblk[T], np.float64) for T in range(wl.n_tensors)] for _ in range(W)]
    mx = np.zeros((W, wl.n_tensors), np.float64)
    for j0, j1, pieces in chunks:
        hm = _host_rows(pin, "m0", m0, j0, j1)
        hg = _host_rows(pin, "g", g, j0, j1)
        torch.cuda.synchronize()
        am, ag = _np(hm), _np(hg, gb)

        def one(task):
            i, (T, a, b) = task
            mp = am[i, a - j0:b - j0]
            gp = ag[i, a - j0:b - j0]
            if wl.agg == "linf":
                mx[i, T] = max(mx[i, T], lco.minf(lco.c_row(wl, mp, gp)))
                return
            k0 = (a - off[T]) // BLOCK
            n = b - a
            P = parts[i][T]
            L.lco_m1_partials(cfg.ref, n, mp.ctypes.data_as(C.c_void_p),
                              gp.ctypes.data_as(C.c_void_p),
                              C.c_void_p(P.ctypes.data + 8 * k0))
        # one task per (worker, tensor piece): a chunk holds at most one
        # piece of each tensor, so no two tasks touch the same pair
        list(pool.map(one, [(i, pc) for i in range(W) for pc in pieces]))
    if wl.agg == "linf":
        return mx
    out = np.empty((W, wl.n_tensors), np.float64)
    for i in range(W):
        for T in range(wl.n_tensors):
            out[i, T] = lco.m1_finalize(parts[i][T], off[T + 1] - off[T])
    return out


def check_step_every_element(wl, lc, theta, m, g, t, P=16, chunk=1 << 22):
    """Run one device step on (theta, m, g) at step t and compare every
    element of theta and m, and every norm, with the oracle."""
    import torch
    tb, gb = wl.theta_dtype == "bf16", wl.grad_dtype == "bf16"
    quant = wl.agg in ("l1", "linf")
    t0 = time.perf_counter()
    th0 = theta.clone()
    m0 = m.clone()
    dbg = None
    if quant:
        dbg = {"m1": torch.zeros((wl.W, wl.n_tensors), dtype=torch.float64, device=m.device)}
    lc.step(theta, m, g, t, dbg)
    torch.cuda.synchronize()
    chunks = column_chunks(wl, chunk)
    pin = Pinned()
    L = lco.lib()
    cfg = lco.OracleCfg(wl)
    with ThreadPoolExecutor(max_workers=P) as pool:
        norms = None
        if quant:
            norms = oracle_norms(wl, m0, g, pin, pool, chunks)
            got = dbg["m1"].cpu().numpy()
            bad = np.argwhere(got.view(np.uint64) != norms.view(np.uint64))
            assert bad.size == 0, f"norms differ at {bad[:5].tolist()} (t={t})"
            _say(wl.name, f"t={t} norms of all {wl.W}x{wl.n_tensors} pairs bit-equal "
                          f"({time.perf_counter() - t0:.1f} s)")
        nref = (C.c_void_p(norms.ctypes.data) if quant else None)
        ncols = 0
        for j0, j1, _ in chunks:
            n = j1 - j0
            ht = _np(_host_vec(pin, "th0", th0, j0, j1), tb)
            hm = _np(_host_rows(pin, "m0", m0, j0, j1))
            hg = _np(_host_rows(pin, "g", g, j0, j1), gb)
            rt = _np(_host_vec(pin, "th1", theta, j0, j1), tb)
            rm = _np(_host_rows(pin, "m1", m, j0, j1))
            torch.cuda.synchronize()
            # the oracle updates its copies in place, P column ranges at once
            per = -(-n // P)
            subs = [(s, min(n, s + per)) for s in range(0, n, per)]

            def run(r):
                a, b = r
                L.lco_step_range(cfg.ref, j0 + a, j0 + b, nref,
                                 C.c_void_p(ht.ctypes.data + a * ht.itemsize),
                                 C.c_void_p(hm.ctypes.data + a * hm.itemsize),
                                 C.c_void_p(hg.ctypes.data + a * hg.itemsize), n, t, None)
            list(pool.map(run, subs))
            _check(pool, f"theta[{j0}:{j1}] t={t}", rt[None, :], ht[None, :], tb)
            _check(pool, f"m[:, {j0}:{j1}] t={t}", rm, hm, False)
            ncols += n
    assert ncols == wl.d
    del th0, m0
    _say(wl.name, f"t={t} every element of theta[{wl.d}] and m[{wl.W}][{wl.d}] equal "
                  f"({time.perf_counter() - t0:.1f} s)")
