"""MI355X (gfx950) Lion Cub / Distributed Lion compressed-update step.

The library (liblioncub.so, C ABI in include/lioncub.h) runs W simulated
data-parallel workers stacked in one GPU's memory: each forms its Lion update
vector, compresses it to a 0/1 sign bitmap or to L1-quantised n-bit codes,
the workers are aggregated by majority vote or integer sum, and the global
sign updates the parameters and each worker's momentum.  `_abi` mirrors the C
entry points; `LionCub` keeps a context and its workspace together;
`StaticStep` runs the allocation-free step with the same options.
"""
from . import _abi, _checks
from ._abi import (AGG_AVG, AGG_L1SUM, AGG_LINFSUM, AGG_VOTE, BF16, F32, TIE_PARITY, TIE_ZERO,
                   LionCubError, lioncub_apply, lioncub_destroy, lioncub_init, lioncub_pack,
                   lioncub_pack_codes, lioncub_profile_begin, lioncub_profile_end,
                   lioncub_quant_l1, lioncub_quant_linf, lioncub_set_stream, lioncub_step,
                   lioncub_step_static, lioncub_strerror, lioncub_unpack_sum,
                   lioncub_unpack_sum_bits, lioncub_vote, lioncub_vote_bits,
                   lioncub_workspace_bytes, make_config)

__all__ = ["LionCub", "StaticStep", "LionCubError", "make_config", "lioncub_workspace_bytes",
           "lioncub_init", "lioncub_set_stream", "lioncub_step", "lioncub_step_static",
           "lioncub_pack", "lioncub_vote",
           "lioncub_quant_l1", "lioncub_quant_linf", "lioncub_vote_bits", "lioncub_apply",
           "lioncub_pack_codes", "lioncub_unpack_sum", "lioncub_unpack_sum_bits",
           "lioncub_profile_begin", "lioncub_profile_end",
           "lioncub_destroy", "lioncub_strerror", "F32", "BF16", "AGG_VOTE", "AGG_L1SUM",
           "AGG_AVG", "AGG_LINFSUM", "TIE_PARITY", "TIE_ZERO"]


def _configure(obj, d, W, tensor_offsets, ld, sync_m, sync_every, theta_dtype, grad_dtype, agg,
               qbits, tie, beta1, beta2, lr, wd, sr_seed):
    """Validate the Python-level options and set obj.cfg (the lioncub_config
    and the host arrays it points to), obj.spec (what the host-side tensor
    checks need) and the plain fields."""
    aggs = {"vote": AGG_VOTE, "l1": AGG_L1SUM, "avg": AGG_AVG, "linf": AGG_LINFSUM}
    if agg not in aggs:
        raise ValueError(f"agg must be one of {sorted(aggs)}, got {agg!r}")
    for name, val, allowed in (("theta_dtype", theta_dtype, ("f32", "bf16")),
                               ("grad_dtype", grad_dtype, ("f32", "bf16")),
                               ("tie", tie, ("parity", "zero"))):
        if val not in allowed:
            raise ValueError(f"{name} must be one of {allowed}, got {val!r}")
    ld = ld if ld is not None else (d + 63) // 64 * 64
    offs = tensor_offsets if tensor_offsets is not None else [0, d]
    obj.cfg = make_config(
        d, ld, W, offs, sync_m=sync_m, sync_every=sync_every,
        theta_dtype=BF16 if theta_dtype == "bf16" else F32,
        grad_dtype=BF16 if grad_dtype == "bf16" else F32,
        agg=aggs[agg], qbits=qbits,
        tie_mode=TIE_ZERO if tie == "zero" else TIE_PARITY,
        beta1=beta1, beta2=beta2, lr=lr, wd=wd, sr_seed=sr_seed)
    obj.d, obj.ld, obj.W, obj.n_tensors = d, ld, W, len(offs) - 1
    obj.agg, obj.sync_every = agg, sync_every
    obj.spec = _checks.Spec(d=d, ld=ld, W=W, n_tensors=len(offs) - 1,
                            theta_dtype=theta_dtype, grad_dtype=grad_dtype, qbits=qbits)


class StaticStep:
    """The allocation-free step (lioncub_step_static) with the same options
    as LionCub: no context, no workspace and no device memory of its own --
    the library's fixed scratch array holds the step's tables and partials.
    For code that may not allocate (e.g. under stream capture).  Each step
    checks its tensors on the host first; calls that overlap on one GPU race
    on the shared array."""

    def __init__(self, d, W, tensor_offsets=None, ld=None, sync_m=None, sync_every=1,
                 theta_dtype="f32", grad_dtype="f32", agg="vote", qbits=0, tie="parity",
                 beta1=0.9, beta2=0.99, lr=1e-4, wd=0.1, sr_seed=0):
        _configure(self, d, W, tensor_offsets, ld, sync_m, sync_every, theta_dtype, grad_dtype,
                   agg, qbits, tie, beta1, beta2, lr, wd, sr_seed)
        nbytes = lioncub_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise LionCubError("lioncub_workspace_bytes", _abi.EINVAL)
        if nbytes > _abi.STATIC_SCRATCH_BYTES:
            raise LionCubError("lioncub_step_static", _abi.ESCRATCH)

    def step(self, theta, m, g, t, stream=None):
        """One step in place on `stream` (a torch.cuda.Stream; default: the
        current stream of theta's device, which must be the current device)."""
        import torch
        _checks.state(self.spec, theta.device, theta, m, g)
        s = stream if stream is not None else torch.cuda.current_stream(theta.device)
        lioncub_step_static(self.cfg, _abi._stream_handle(s), theta, m, g, t)


class LionCub:
    """One context: configuration, a torch-allocated workspace, a stream.

    theta: [d] fp32/bf16, m: [W][ld] fp32, g: [W][ld] fp32/bf16, all torch
    tensors on the device; updated in place by step()."""

    def __init__(self, d, W, tensor_offsets=None, ld=None, sync_m=None, sync_every=1,
                 theta_dtype="f32", grad_dtype="f32", agg="vote", qbits=0, tie="parity",
                 beta1=0.9, beta2=0.99, lr=1e-4, wd=0.1, sr_seed=0, device="cuda", stream=None):
        import torch
        _configure(self, d, W, tensor_offsets, ld, sync_m, sync_every, theta_dtype, grad_dtype,
                   agg, qbits, tie, beta1, beta2, lr, wd, sr_seed)
        nbytes = lioncub_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise LionCubError("lioncub_workspace_bytes", _abi.EINVAL)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.device = self.workspace.device
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        self.ctx = lioncub_init(self.cfg, _abi._stream_handle(self.stream), self.workspace)

    def set_stream(self, stream):
        """Enqueue later calls on `stream` (a torch.cuda.Stream), e.g. the
        capturing stream of a torch.cuda.graph."""
        lioncub_set_stream(self.ctx, _abi._stream_handle(stream))
        self.stream = stream

    # Every method checks its tensors on the host (_checks) before passing
    # their pointers: the C ABI cannot see a buffer's extent.

    def step(self, theta, m, g, t, debug=None):
        _checks.step(self.spec, self.device, theta, m, g, debug)
        lioncub_step(self.ctx, theta, m, g, t, debug)

    def capture(self, theta, m, gs, t0):
        """Capture len(gs) consecutive steps (step t0 + k reads gs[k]) into a
        torch.cuda.CUDAGraph and return it; graph.replay() runs them.

        A step depends on t only through t's parity (zeros and ties) and
        t % sync_every (averaging steps), so when K = len(gs) is a multiple
        of lcm(2, sync_every), replaying the window is exactly the next K
        steps: replay r runs steps t0 + r*K .. t0 + r*K + K - 1.  The
        max-norm baseline draws its random numbers from the full t and is
        refused.  The graph keeps the tensors it was captured with; the
        caller refills gs between replays.  Profiling must be off."""
        import math

        import torch
        K = len(gs)
        period = 2 * self.sync_every // math.gcd(2, self.sync_every)
        if self.agg == "linf":
            raise ValueError("capture: the max-norm baseline's draws depend on the full step index")
        if getattr(self, "_profiling", False):
            raise ValueError("capture: profiling is on (its events would be recorded into the graph)")
        if K == 0 or K % period:
            raise ValueError(f"capture: the number of steps must be a multiple of {period}")
        for g in gs:
            _checks.state(self.spec, self.device, theta, m, g)
        graph = torch.cuda.CUDAGraph()
        prev = self.stream
        try:
            with torch.cuda.graph(graph):
                self.set_stream(torch.cuda.current_stream())
                for k, g in enumerate(gs):
                    lioncub_step(self.ctx, theta, m, g, t0 + k, None)
        finally:
            self.set_stream(prev)
        return graph

    def pack(self, x, t, bits):
        _checks.pack(self.spec, self.device, x, bits)
        lioncub_pack(self.ctx, x, t, bits)

    def vote(self, bits, t, counts=None, sign=None):
        _checks.vote(self.spec, self.device, bits, counts, sign)
        lioncub_vote(self.ctx, bits, t, counts, sign)

    def quant_l1(self, x, codes, m1=None):
        _checks.quant(self.spec, self.device, x, codes, m1)
        lioncub_quant_l1(self.ctx, x, codes, m1)

    def quant_linf(self, x, t, codes, minf=None):
        _checks.quant(self.spec, self.device, x, codes, minf)
        lioncub_quant_linf(self.ctx, x, t, codes, minf)

    def vote_bits(self, bits, t, sign_bits, zero_bits=None):
        _checks.vote_bits(self.spec, self.device, bits, sign_bits, zero_bits)
        lioncub_vote_bits(self.ctx, bits, t, sign_bits, zero_bits)

    def apply(self, theta, m, g, t, sign_bits, zero_bits=None):
        _checks.apply(self.spec, self.device, theta, m, g, sign_bits, zero_bits)
        lioncub_apply(self.ctx, theta, m, g, t, sign_bits, zero_bits)

    def pack_codes(self, codes, wire):
        _checks.pack_codes(self.spec, self.device, codes, wire)
        lioncub_pack_codes(self.ctx, codes, wire)

    def unpack_sum(self, wire, sums=None, sign=None):
        _checks.unpack_sum(self.spec, self.device, wire, sums, sign)
        lioncub_unpack_sum(self.ctx, wire, sums, sign)

    def unpack_sum_bits(self, wire, sign_bits, zero_bits=None):
        _checks.unpack_sum_bits(self.spec, self.device, wire, sign_bits, zero_bits)
        lioncub_unpack_sum_bits(self.ctx, wire, sign_bits, zero_bits)

    def profile_begin(self, capacity):
        lioncub_profile_begin(self.ctx, capacity)
        self._profiling = True

    def profile_end(self):
        out = lioncub_profile_end(self.ctx)
        self._profiling = False
        return out

    def close(self):
        if getattr(self, "ctx", None) is not None:
            lioncub_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
