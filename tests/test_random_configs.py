"""Seeded random configurations of the forward against the fp64 oracle (GPU).

The hand-written parity cases cover each feature on its own; these draws mix
them: dtype (bf16 / fp32), head dim, every chunk that dtype supports, ragged T,
batch and heads, with or without h0, per-key-dim or scalar gates, gate
families (ordinary, strong decay past the exact-path guard, 1% spikes of
-200, zero) and the segment target (one segment per head up to many).  Every
output element and every final state is compared with the oracle's token
recurrence, normalised over the whole tensor, at the forward's bar (1e-2 for
bf16, 1e-3 for fp32).  The draws come from a fixed seed, so a failure names a
reproducible case.
"""

import dataclasses
import random
import sys

import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import WORKLOADS, make_inputs
from wholecheck import select_f64, whole_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 1e-2, "f32": 1e-3}
CHUNKS = {"bf16": [32, 64, 128], "f32": [32, 64]}


def _draws(n=24, seed=20261203):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        dtype = rng.choice(["bf16", "bf16", "f32"])
        out.append(dict(
            idx=i, dtype=dtype, D=rng.choice([64, 128]), chunk=rng.choice(CHUNKS[dtype]),
            B=rng.choice([1, 2]), H=rng.choice([1, 2, 3]), T=rng.randint(1, 1500),
            h0=rng.random() < 0.5, scalar=rng.random() < 0.3,
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
def test_random_configuration(c):
    _say(f"[random] {c}")
    base = WORKLOADS["tiny_f32"] if c["dtype"] == "f32" else WORKLOADS["prefill_4k"]
    wl = dataclasses.replace(base, D=c["D"], scalar_gate=c["scalar"])
    gate = "ls16" if c["gate"] == "spikes" else c["gate"]
    x = make_inputs(wl, B=c["B"], H=c["H"], T=c["T"], seed=c["seed"], gate=gate,
                    h0_std=0.3 if c["h0"] else None)
    if c["gate"] == "spikes":
        gen = torch.Generator().manual_seed(c["seed"] + 1)
        spikes = torch.rand(x["g"].shape, generator=gen) < 0.01
        x["g"] = torch.where(spikes, torch.full_like(x["g"], -200.0), x["g"])
    scale = c["D"] ** -0.5
    gla.set_tuning(c["target"], 0)
    d = {n: (None if x[n] is None else x[n].to(DEV)) for n in ("q", "k", "v", "g", "h0")}
    if c["scalar"]:
        fn = gla.gla_fwd_scalar_f32 if c["dtype"] == "f32" else gla.gla_fwd_scalar
    else:
        fn = gla.gla_fwd_f32 if c["dtype"] == "f32" else gla.gla_fwd
    o, hf = fn(d["q"], d["k"], d["v"], d["g"], d["h0"], chunk=c["chunk"], scale=scale, want_final=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    hf = hf.cpu().numpy()
    B, H, T = c["B"], c["H"], c["T"]

    def ref(sel):
        f = select_f64(x, ("q", "k", "v", "g", "h0"), sel)
        if c["scalar"]:
            ro, rh = oracle.scalar_gate_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], scale)
        else:
            ro, rh, _ = oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], scale)
        return {"o": ro, "h_final": rh}

    errs = whole_errors({"o": o, "h_final": hf}, ref, B, H, T)
    _say(f"    output err {errs['o']:.3e}, h_final err {errs['h_final']:.3e} (tol {TOL[c['dtype']]:g})")
    assert errs["o"] <= TOL[c["dtype"]]
    assert errs["h_final"] <= TOL[c["dtype"]]
