"""Workload descriptions: shapes, tensor lists, dtypes and hyperparameters.

Shared by the tests, the benchmark and the smoke check.  Holds no arithmetic
of the method itself: only sizes, flags and the numbers the workloads fix.

The GPT tensor lists follow the GPT-2 layout (token embedding, learned
positions over a 1024-token context, L blocks of 12 tensors each, final
LayerNorm) with the output projection tied to the token embedding; the
vocabulary is 50257.  These are the model shapes of the GPT experiments on the
Lion Cub pages (GPT 350M-1558M on OpenWebText) and of the D-Lion GPT2++ 760M
run; with a tied head the 12x768, 24x1536 and 24x2048 models have the 124M,
760M and 1.3B sizes the workloads name.
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional

VOCAB = 50257
N_CTX = 1024


def gpt_tensors(n_layer: int, hidden: int, vocab: int = VOCAB, n_ctx: int = N_CTX):
    """(name, numel) list of a GPT-2-layout model with a tied head."""
    h = hidden
    out = [("wte", vocab * h), ("wpe", n_ctx * h)]
    for l in range(n_layer):
        p = f"h{l}."
        out += [
            (p + "ln_1.w", h), (p + "ln_1.b", h),
            (p + "attn.c_attn.w", h * 3 * h), (p + "attn.c_attn.b", 3 * h),
            (p + "attn.c_proj.w", h * h), (p + "attn.c_proj.b", h),
            (p + "ln_2.w", h), (p + "ln_2.b", h),
            (p + "mlp.c_fc.w", h * 4 * h), (p + "mlp.c_fc.b", 4 * h),
            (p + "mlp.c_proj.w", 4 * h * h), (p + "mlp.c_proj.b", h),
        ]
    out += [("ln_f.w", h), ("ln_f.b", h)]
    return out


@dataclass
class Workload:
    name: str
    tensors: List[tuple]              # (name, numel), concatenated in order
    W: int
    agg: str = "vote"                 # "vote" | "l1" | "avg" | "linf"
    qbits: int = 0                    # n of Eq. (1) on the L1 / max-norm paths
    tie: str = "parity"               # "parity" | "zero"
    theta_dtype: str = "f32"          # "f32" | "bf16"
    grad_dtype: str = "f32"           # "f32" | "bf16"
    sync_names: tuple = ()            # tensors whose momentum is averaged
    sync_every: int = 1
    beta1: float = 0.9
    beta2: float = 0.99
    lr: float = 1e-4
    wd: float = 0.1
    steps: int = 5
    seed: int = 0
    theta_std: float = 0.02
    m_std: float = 1e-3
    g_nu: float = 3.0                 # Student-t degrees of freedom
    g_scale: float = 1e-3
    g_tensor_scale: Optional[tuple] = None  # (lo, hi): per-tensor log-uniform scale
    ld_pad: int = 0                   # extra elements of row padding (multiple of 64)
    sr_seed: int = 0x5EED             # key of the stochastic-rounding generator

    @property
    def d(self) -> int:
        return sum(n for _, n in self.tensors)

    @property
    def ld(self) -> int:
        return (self.d + 63) // 64 * 64 + self.ld_pad

    @property
    def offsets(self) -> List[int]:
        off = [0]
        for _, n in self.tensors:
            off.append(off[-1] + n)
        return off

    @property
    def n_tensors(self) -> int:
        return len(self.tensors)

    @property
    def sync_flags(self) -> List[int]:
        return [1 if nm in self.sync_names else 0 for nm, _ in self.tensors]

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def flat(name: str, d: int, **kw) -> Workload:
    return Workload(name=name, tensors=[("flat", d)], **kw)


# The five workloads.  Hyperparameters the descriptions leave open reuse those
# of the first (beta1 0.9, beta2 0.99, lr 1e-4, wd 0.1, seed 0; theta ~ N(0,
# 0.02), m ~ N(0, 1e-3)).
FLAT_1M_W4_VOTE = flat("flat-1M-w4-vote", 1_048_576, W=4, agg="vote", steps=10)

GPT2_124M_W8_VOTE = Workload(
    name="gpt2-124M-w8-vote", tensors=gpt_tensors(12, 768), W=8, agg="vote",
    steps=5, g_tensor_scale=(1e-4, 1e-2))

FLAT_350M_W16_L1Q4 = flat("flat-350M-w16-l1q4", 350_000_000, W=16, agg="l1",
                          qbits=4, steps=5, g_nu=2.5)

GPT_760M_W8_VOTE_SYNC = Workload(
    name="gpt-760M-w8-vote-bf16-syncemb", tensors=gpt_tensors(24, 1536), W=8,
    agg="vote", theta_dtype="bf16", grad_dtype="bf16", sync_names=("wte", "wpe"),
    sync_every=1, steps=3)

GPT_1B3_W8_L1Q8 = Workload(
    name="gpt-1.3B-w8-l1q8-bf16g", tensors=gpt_tensors(24, 2048), W=8, agg="l1",
    qbits=8, grad_dtype="bf16", steps=3)

ALL = [FLAT_1M_W4_VOTE, GPT2_124M_W8_VOTE, FLAT_350M_W16_L1Q4,
       GPT_760M_W8_VOTE_SYNC, GPT_1B3_W8_L1Q8]
BY_NAME = {w.name: w for w in ALL}


def shrink(wl: Workload, max_elems_per_tensor: int, max_tensors: Optional[int] = None,
           name_suffix: str = "-small") -> Workload:
    """Same structure, smaller tensors: every tensor capped (sizes kept
    multiples of 64) and optionally only the first tensors kept, so the
    oracle finishes in seconds while blocks, tails and tensor boundaries are
    all still exercised."""
    ts = []
    for nm, n in wl.tensors[: max_tensors or len(wl.tensors)]:
        m = min(n, max_elems_per_tensor)
        ts.append((nm, m))
    return replace(wl, name=wl.name + name_suffix, tensors=ts)
