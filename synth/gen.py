"""Seeded synthetic inputs: parameters, per-worker momenta and gradients.

Shared by the tests, the benchmark and the smoke check; holds none of the
method's arithmetic.  The value distributions follow the pages' description of
Lion update vectors (Lion Cub, Figure 3: Laplace-like, heavy-tailed, maximum
far above the mean): gradients are Student-t scaled, parameters and momenta
Gaussian.

Host generator: NumPy's Philox counter-based generator, keyed by (seed,
stream, step, worker), so a value depends only on its key and index, never on
chunking.  Values are drawn in fp64, rounded to fp32 (round-to-nearest-even),
then to bf16 (round-to-nearest-even, via torch) where a workload stores bf16.

Device generator (full-size workloads only; the host would take minutes per
step): torch's seeded CUDA generator with the same keys, same distributions.
It never feeds a value to the oracle that the oracle did not also see: tests
that use it download the very buffers the GPU consumed.
"""
import math

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

STREAM_THETA, STREAM_M, STREAM_G, STREAM_SCALE = 1, 2, 3, 4


def _key(seed, stream, step, worker):
    return np.array([seed & (2**64 - 1),
                     (stream << 56) | ((step & 0xFFFFFF) << 32) | (worker & 0xFFFFFFFF)],
                    dtype=np.uint64)


def rng(seed, stream, step=0, worker=0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=_key(seed, stream, step, worker)))


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even, via torch."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return to_bf16_bits(x32) if dtype == "bf16" else x32


def tensor_scales(wl) -> np.ndarray:
    """Per-tensor gradient scale: log-uniform in wl.g_tensor_scale, drawn once."""
    if wl.g_tensor_scale is None:
        return np.full(wl.n_tensors, wl.g_scale)
    lo, hi = wl.g_tensor_scale
    u = rng(wl.seed, STREAM_SCALE).random(wl.n_tensors)
    return np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def host_theta(wl) -> np.ndarray:
    """theta[d]: fp32 array, or uint16 bf16 bits."""
    x = rng(wl.seed, STREAM_THETA).normal(0.0, wl.theta_std, wl.d)
    return _store(x, wl.theta_dtype)


def host_m(wl) -> np.ndarray:
    """m[W][ld] fp32; the row padding [d, ld) is zero."""
    m = np.zeros((wl.W, wl.ld), dtype=np.float32)
    for i in range(wl.W):
        m[i, : wl.d] = rng(wl.seed, STREAM_M, 0, i).normal(0.0, wl.m_std, wl.d).astype(np.float32)
    return m


def host_g(wl, step: int) -> np.ndarray:
    """g[W][ld] for step `step` (fresh per step and worker); padding zero."""
    dt = np.uint16 if wl.grad_dtype == "bf16" else np.float32
    g = np.zeros((wl.W, wl.ld), dtype=dt)
    sc = tensor_scales(wl)
    off = wl.offsets
    per_elem = np.repeat(sc, np.diff(off))
    for i in range(wl.W):
        x = rng(wl.seed, STREAM_G, step, i).standard_t(wl.g_nu, wl.d) * per_elem
        g[i, : wl.d] = _store(x, wl.grad_dtype)
    return g


# ------------------------------------------------------------------ device --

def _torch_gen(seed, stream, step, worker, device):
    k = _key(seed, stream, step, worker)
    s = int((int(k[0]) * 0x9E3779B97F4A7C15 + int(k[1])) & (2**63 - 1))
    return torch.Generator(device=device).manual_seed(s)


def _dev_store(x: "torch.Tensor", dtype: str) -> "torch.Tensor":
    x32 = x.to(torch.float32)
    return x32.to(torch.bfloat16) if dtype == "bf16" else x32


def _dev_student_t(n, nu, gen, device, chunk=1 << 26):
    out = torch.empty(n, dtype=torch.float64, device=device)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        z = torch.randn(b - a, dtype=torch.float64, device=device, generator=gen)
        alpha = torch.full((b - a,), nu / 2.0, dtype=torch.float64, device=device)
        chi2 = 2.0 * torch._standard_gamma(alpha, generator=gen)
        out[a:b] = z * torch.sqrt(nu / chi2)
        del z, alpha, chi2
    return out


def device_theta(wl, device="cuda"):
    gen = _torch_gen(wl.seed, STREAM_THETA, 0, 0, device)
    out = torch.empty(wl.d, dtype=torch.bfloat16 if wl.theta_dtype == "bf16" else torch.float32,
                      device=device)
    chunk = 1 << 26
    for a in range(0, wl.d, chunk):
        b = min(wl.d, a + chunk)
        x = torch.randn(b - a, dtype=torch.float64, device=device, generator=gen) * wl.theta_std
        out[a:b] = _dev_store(x, wl.theta_dtype)
    return out


def device_m(wl, device="cuda"):
    m = torch.zeros((wl.W, wl.ld), dtype=torch.float32, device=device)
    chunk = 1 << 26
    for i in range(wl.W):
        gen = _torch_gen(wl.seed, STREAM_M, 0, i, device)
        for a in range(0, wl.d, chunk):
            b = min(wl.d, a + chunk)
            m[i, a:b] = (torch.randn(b - a, dtype=torch.float64, device=device, generator=gen)
                         * wl.m_std).to(torch.float32)
    return m


def fill_device_g(wl, step, out):
    """Write g for `step` into out[W][ld] (torch fp32 or bf16 on the GPU)."""
    sc = torch.from_numpy(tensor_scales(wl)).to(out.device)
    off = wl.offsets
    per = torch.repeat_interleave(sc, torch.tensor(np.diff(off), device=out.device))
    out[:, wl.d:].zero_()
    for i in range(wl.W):
        gen = _torch_gen(wl.seed, STREAM_G, step, i, out.device)
        chunk = 1 << 26
        for a in range(0, wl.d, chunk):
            b = min(wl.d, a + chunk)
            x = _dev_student_t(b - a, wl.g_nu, gen, out.device, chunk) * per[a:b]
            out[i, a:b] = _dev_store(x, wl.grad_dtype)
    return out


def device_g(wl, step, device="cuda"):
    dt = torch.bfloat16 if wl.grad_dtype == "bf16" else torch.float32
    out = torch.empty((wl.W, wl.ld), dtype=dt, device=device)
    return fill_device_g(wl, step, out)
