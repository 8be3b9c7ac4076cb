"""Seeded synthetic inputs for the gated linear attention prefill forward.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the HIP path and the CPU oracle receive exactly the tensors
made here (the oracle after an exact widening to float64).

Recipe (one CPU ``torch.Generator`` per call, draw order q, k, v, gate
normal, h0; values drawn in float32):

* q, v ~ N(0, 1).
* k ~ N(0, 1), then either scaled by 1/sqrt(K) ("scaled") or L2-normalised
  over the key dim per token ("l2", eps 1e-6).
* gate g, one value per key dim and token, float32:
  "ls16"  = logsigmoid(N(0, 1)) / 16,
  "ls41"  = logsigmoid(N(4, 1))  (gates close to 1: long memory),
  "zero"  = 0 (no decay: reduces to causal (Q K^T * M) V),
  "const:<x>" = the constant x (extreme-gate tests, e.g. -30 or -1e4).
* h0 ~ N(0, std) in float32 when the workload asks for one, else absent.
* For bf16 workloads q, k, v are rounded to bfloat16 (round to nearest even,
  by torch); g and h0 stay float32.

The pages measure on synthetic shapes only (B, H, T, D sweeps); no dataset
stands behind these numbers, and none is used here.

Scalar-gate workloads (SCALAR_WORKLOADS) draw g with shape [B,H,T], one
log-decay per token and head (same distributions), for the scalar-gate
variant of the forward.

Backward inputs (make_grad_inputs): the loss gradients do ~ N(0, 1) (in the
workload's dtype) and dh_final ~ N(0, 0.1) (fp32), from a generator of their
own seeded with the workload seed + 1000.

Gated delta rule workloads (GDN_WORKLOADS, make_gdn_inputs): q and k
L2-normalised per token (the delta rule's convention), v ~ N(0, 1), all
three rounded to bf16; g = logsigmoid(N(0, 1)) / 16 and beta = sigmoid(N(0,
1)), fp32, one per token and head; h0 ~ N(0, std) when asked.  Draw order
q, k, v, g normal, beta normal, h0, from one generator per call.

Decode workloads (DECODE_WORKLOADS) draw the same way with T = 1: one new
token per (batch, head) and a carried fp32 state drawn as h0.  The pages do
not measure decode; the batch is sized so that the state of one step
(B*H*D*D*4 bytes, 256 MiB at B=256, H=16, D=128) is as large as the MI355X
Infinity Cache, and two such sets alternate in the benchmark.
"""

from __future__ import annotations

import dataclasses
import math

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int            # K == V == D
    dtype: str        # "bf16" or "f32" for q, k, v, o
    k_mode: str       # "scaled" or "l2"
    gate: str         # see module docstring
    h0_std: float | None
    want_final: bool
    chunk: int | None  # None: the library's default chunk
    seed: int
    scalar_gate: bool = False   # g is [B,H,T]: one log-decay per token and head

    @property
    def scale(self) -> float:
        return self.D ** -0.5

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads: a tiny fp32 case, three H=16 D=128 bf16 prefill shapes
# and a long-sequence case with gates near 1 and a nonzero initial state.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 256, 64, "f32", "scaled", "ls16", None, True, 64, 0),
    "prefill_4k": Workload("prefill_4k", 1, 16, 4096, 128, "bf16", "l2", "ls16", None, False, None, 1),
    "prefill_16k": Workload("prefill_16k", 1, 16, 16384, 128, "bf16", "l2", "ls16", None, True, None, 2),
    "batch16_4k": Workload("batch16_4k", 16, 16, 4096, 128, "bf16", "l2", "ls16", None, False, None, 3),
    "long_128k": Workload("long_128k", 1, 16, 131072, 128, "bf16", "l2", "ls41", 0.02, True, None, 4),
}


# Scalar gate: the prefill_16k shape with one gate per token and head.
SCALAR_WORKLOADS = {
    "prefill_16k_scalar": Workload("prefill_16k_scalar", 1, 16, 16384, 128, "bf16", "l2", "ls16",
                                   None, True, None, 6, scalar_gate=True),
}

# Gated delta rule: 16 sequences x 16 heads of 4K tokens (one work-group per
# sequence-head fills the GPU), and a long single sequence.
GDN_WORKLOADS = {
    "gdn_b16_4k": Workload("gdn_b16_4k", 16, 16, 4096, 128, "bf16", "l2", "ls16", None, True, 64, 7),
    "gdn_16k": Workload("gdn_16k", 1, 16, 16384, 128, "bf16", "l2", "ls16", None, True, 64, 8),
}

# Decode: B sequences x H heads each take one step against a carried state.
DECODE_WORKLOADS = {
    "decode_b256": Workload("decode_b256", 256, 16, 1, 128, "bf16", "l2", "ls16", 0.05, True, None, 5),
}


def _gate(kind: str, shape, gen) -> torch.Tensor:
    if kind == "ls16":
        return F.logsigmoid(torch.randn(shape, generator=gen)) / 16.0
    if kind == "ls41":
        return F.logsigmoid(torch.randn(shape, generator=gen) + 4.0)
    # the normal draw is still taken so the h0 draw does not depend on the gate
    torch.randn(shape, generator=gen)
    if kind == "zero":
        return torch.zeros(shape)
    if kind.startswith("const:"):
        return torch.full(shape, float(kind.split(":", 1)[1]))
    raise ValueError(f"unknown gate kind {kind!r}")


def make_inputs(wl: Workload, *, B=None, H=None, T=None, gate=None, seed=None,
                h0_std="default"):
    """Draw (q, k, v, g, h0) on the CPU for workload ``wl``.

    Overrides shrink or vary the shape (parity cases) while keeping the
    workload's distributions.  Returns a dict of CPU tensors; ``h0`` is None
    when the workload has no initial state.
    """
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    T = wl.T if T is None else T
    D = wl.D
    gate = wl.gate if gate is None else gate
    seed = wl.seed if seed is None else seed
    std = wl.h0_std if h0_std == "default" else h0_std
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    shape = (B, H, T, D)
    q = torch.randn(shape, generator=gen)
    k = torch.randn(shape, generator=gen)
    v = torch.randn(shape, generator=gen)
    g = _gate(gate, (B, H, T) if wl.scalar_gate else shape, gen)
    if wl.k_mode == "l2":
        k = F.normalize(k, dim=-1, eps=1e-6)
    elif wl.k_mode == "scaled":
        k = k * (1.0 / math.sqrt(D))
    else:
        raise ValueError(wl.k_mode)
    h0 = None
    if std is not None:
        h0 = torch.randn((B, H, D, D), generator=gen) * std
    if wl.dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "g": g.float().contiguous(), "h0": None if h0 is None else h0.contiguous()}


def make_gdn_inputs(wl: Workload, *, B=None, H=None, T=None, gate=None, seed=None,
                    h0_std="default", beta=None):
    """Draw (q, k, v, g, beta, h0) for the gated delta rule on workload ``wl``.
    ``gate`` overrides g as for make_inputs; ``beta`` may fix beta to a constant."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    T = wl.T if T is None else T
    D = wl.D
    gate = wl.gate if gate is None else gate
    seed = wl.seed if seed is None else seed
    std = wl.h0_std if h0_std == "default" else h0_std
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    shape = (B, H, T, D)
    q = F.normalize(torch.randn(shape, generator=gen), dim=-1, eps=1e-6)
    k = F.normalize(torch.randn(shape, generator=gen), dim=-1, eps=1e-6)
    v = torch.randn(shape, generator=gen)
    g = _gate(gate, (B, H, T), gen)
    b = torch.sigmoid(torch.randn((B, H, T), generator=gen))
    if beta is not None:
        b = torch.full((B, H, T), float(beta))
    h0 = None
    if std is not None:
        h0 = torch.randn((B, H, D, D), generator=gen) * std
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "g": g.float().contiguous(), "beta": b.float().contiguous(),
            "h0": None if h0 is None else h0.contiguous()}


def make_grad_inputs(wl: Workload, *, B=None, H=None, T=None, seed=None, dh_final=True):
    """Draw the loss gradients (do, dh_final) for a backward of workload ``wl``."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    T = wl.T if T is None else T
    seed = (wl.seed if seed is None else seed) + 1000
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    do = torch.randn((B, H, T, wl.D), generator=gen)
    dhf = torch.randn((B, H, wl.D, wl.D), generator=gen) * 0.1 if dh_final else None
    if wl.dtype == "bf16":
        do = do.to(torch.bfloat16)
    return {"do": do.contiguous(), "dh_final": None if dhf is None else dhf.contiguous()}


def to_f64_numpy(t):
    """Exact widening of a CPU tensor (bf16 or fp32) to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
