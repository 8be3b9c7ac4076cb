"""Seeded random configurations of the backward against the fp64 oracle (GPU).

Draws mix dtype, head dim, the backward's chunks (32, 64; fp32 at K = 128:
32), ragged T, batch and heads, h0 and dh_final present or absent, gate
families (ordinary, strong decay past the exact-path guard, 1% spikes of
-200, zero) and the segment target.  Every element of dq, dk, dv, dg and dh0
is compared with the oracle's reverse-mode chain rule, normalised over each
whole tensor, at the backward's bar (1e-2 bf16, 1e-3 fp32).  The draws come
from a fixed seed, so a failure names a reproducible case.
"""

import dataclasses
import random
import sys

import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import WORKLOADS, make_grad_inputs, make_inputs
from wholecheck import select_f64, whole_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 1e-2, "f32": 1e-3}
NAMES = ("dq", "dk", "dv", "dg", "dh0")


def _chunks(dtype, D):
    return [32] if (dtype == "f32" and D == 128) else [32, 64]


def _draws(n=12, seed=20261204):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        dtype = rng.choice(["bf16", "bf16", "f32"])
        D = rng.choice([64, 128])
        out.append(dict(
            idx=i, dtype=dtype, D=D, chunk=rng.choice(_chunks(dtype, D)),
            B=rng.choice([1, 2]), H=rng.choice([1, 2]), T=rng.randint(1, 800),
            h0=rng.random() < 0.5, dhf=rng.random() < 0.5,
            gate=rng.choice(["ls16", "ls16", "const:-2", "spikes", "zero"]),
            target=rng.choice([0, 1, 6, 64]), seed=rng.randint(0, 10**6)))
    return out


DRAWS = _draws()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _default_tuning():
    gla.set_tuning(0, 0)
    yield
    gla.set_tuning(0, 0)


@pytest.mark.parametrize("c", DRAWS, ids=[f"draw{c['idx']}" for c in DRAWS])
def test_random_backward(c):
    _say(f"[random bwd] {c}")
    base = WORKLOADS["tiny_f32"] if c["dtype"] == "f32" else WORKLOADS["prefill_4k"]
    wl = dataclasses.replace(base, D=c["D"])
    gate = "ls16" if c["gate"] == "spikes" else c["gate"]
    B, H, T = c["B"], c["H"], c["T"]
    x = make_inputs(wl, B=B, H=H, T=T, seed=c["seed"], gate=gate, h0_std=0.3 if c["h0"] else None)
    if c["gate"] == "spikes":
        gen = torch.Generator().manual_seed(c["seed"] + 1)
        spikes = torch.rand(x["g"].shape, generator=gen) < 0.01
        x["g"] = torch.where(spikes, torch.full_like(x["g"], -200.0), x["g"])
    gr = make_grad_inputs(wl, B=B, H=H, T=T)
    if not c["dhf"]:
        gr["dh_final"] = None
    gla.set_tuning(c["target"], 0)
    d = {n: (None if x[n] is None else x[n].to(DEV)) for n in ("q", "k", "v", "g", "h0")}
    do = gr["do"].to(DEV)
    dhf = None if gr["dh_final"] is None else gr["dh_final"].to(DEV)
    fn = gla.gla_bwd_f32 if c["dtype"] == "f32" else gla.gla_bwd
    got = [t.float().cpu().numpy() for t in fn(d["q"], d["k"], d["v"], d["g"], d["h0"], do, dhf,
                                               chunk=c["chunk"])]
    torch.cuda.synchronize()
    src = dict(x)
    src["do"], src["dhf"] = gr["do"], gr["dh_final"]
    scale = c["D"] ** -0.5

    def ref(sel):
        f = select_f64(src, ("q", "k", "v", "g", "h0", "do", "dhf"), sel)
        r = oracle.token_recurrence_backward(f["q"], f["k"], f["v"], f["g"], f["h0"], f["do"], f["dhf"], scale)
        return dict(zip(NAMES, r))

    errs = whole_errors(dict(zip(NAMES, got)), ref, B, H, T)
    _say("    " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f"  (tol {TOL[c['dtype']]:g})")
    bad = {n: e for n, e in errs.items() if not e <= TOL[c["dtype"]]}
    assert not bad, bad
