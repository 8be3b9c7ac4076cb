"""GPU parity of the scalar-gate forward (include/gla_scalar.h): g is [B,H,T],
one log-decay per token and head.  Compared with the fp64 oracle
(oracle.scalar_gate_recurrence) element by element; bar as for the
per-key-dim forward: max|x - x_ref| / max|x_ref| <= 1e-2 for bf16 output,
<= 1e-3 for fp32, the same for the final state, and no NaN/Inf.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import (SCALAR_WORKLOADS, WORKLOADS, make_inputs,
                                                    to_f64_numpy)
from wholecheck import select_f64, whole_errors

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_F32 = 1e-3
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def nerr(out, ref):
    out = np.asarray(out, dtype=np.float64)
    return float(np.max(np.abs(out - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


@pytest.fixture(autouse=True)
def _default_tuning():
    gla.set_tuning(0, 0)
    yield
    gla.set_tuning(0, 0)


def _wl(dtype, D):
    base = WORKLOADS["tiny_f32"] if dtype == "f32" else WORKLOADS["prefill_4k"]
    return dataclasses.replace(base, D=D, scalar_gate=True)


def gpu_run(x, *, fp32=False, chunk=0, want_final=True):
    d = {n: (None if x[n] is None else x[n].to(DEV)) for n in ("q", "k", "v", "g", "h0")}
    fn = gla.gla_fwd_scalar_f32 if fp32 else gla.gla_fwd_scalar
    o, hf = fn(d["q"], d["k"], d["v"], d["g"], d["h0"], chunk=chunk, want_final=want_final)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (None if hf is None else hf.cpu().numpy())


def check(x, o, hf, tol):
    """Every output element and final state against the oracle (in groups of
    sequences), normalised over the whole tensor."""
    B, H, T, K = x["q"].shape
    scale = K ** -0.5

    def ref(sel):
        f = select_f64(x, ("q", "k", "v", "g", "h0"), sel)
        ro, rh = oracle.scalar_gate_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], scale)
        return {"o": ro, "h_final": rh}

    errs = whole_errors({"o": o, "h_final": hf}, ref, B, H, T)
    say(f"    output err {errs['o']:.3e} (tol {tol:g})"
        + (f", h_final err {errs['h_final']:.3e}" if "h_final" in errs else ""))
    assert errs["o"] <= tol
    if "h_final" in errs:
        assert errs["h_final"] <= tol


@pytest.mark.parametrize("gate", ["ls16", "zero", "const:-30"])
@pytest.mark.parametrize("chunk", [64, 32])
def test_f32_tiny(gate, chunk):
    say(f"[scalar f32] D=64 T=256 gate={gate} chunk={chunk}")
    x = make_inputs(_wl("f32", 64), gate=gate, h0_std=0.5)
    o, hf = gpu_run(x, fp32=True, chunk=chunk)
    check(x, o, hf, TOL_F32)


@pytest.mark.parametrize("chunk", [32, 64])
def test_f32_head_dim_128(chunk):
    say(f"[scalar f32] D=128 T=200 chunk={chunk}")
    x = make_inputs(_wl("f32", 128), T=200, H=2, h0_std=0.3)
    o, hf = gpu_run(x, fp32=True, chunk=chunk)
    check(x, o, hf, TOL_F32)


SMALL = [
    # (B, H, T, D, chunk, h0)
    (1, 2, 1, 128, 64, True),
    (2, 3, 63, 128, 64, False),
    (2, 2, 65, 128, 64, True),
    (1, 3, 200, 128, 32, True),
    (2, 2, 1000, 128, 64, True),
    (1, 2, 777, 64, 64, True),
    (1, 2, 300, 64, 32, False),
    (2, 2, 129, 128, 128, True),
    (2, 2, 1000, 128, 128, True),
    (1, 2, 777, 64, 128, True),
]


@pytest.mark.parametrize("B,H,T,D,chunk,h0", SMALL)
def test_bf16_small_shapes(B, H, T, D, chunk, h0):
    say(f"[scalar bf16] B={B} H={H} T={T} D={D} chunk={chunk} h0={h0}")
    x = make_inputs(_wl("bf16", D), B=B, H=H, T=T, seed=T + D + 1, h0_std=0.5 if h0 else None)
    o, hf = gpu_run(x, chunk=chunk)
    check(x, o, hf, TOL_BF16)


@pytest.mark.parametrize("target", [1, 7, 100000])
def test_bf16_segment_splits(target):
    """1 .. N segments: the scalar-gate state pass and the scan are exercised."""
    say(f"[scalar segments] target_wgs={target}")
    x = make_inputs(_wl("bf16", 128), B=1, H=2, T=1000, seed=21, h0_std=0.3)
    gla.set_tuning(target, 0)
    o, hf = gpu_run(x)
    check(x, o, hf, TOL_BF16)


@pytest.mark.parametrize("gate", ["const:-30", "const:-10000", "ls41"])
def test_bf16_extreme_gates(gate):
    say(f"[scalar extreme gates] {gate}")
    x = make_inputs(_wl("bf16", 128), B=1, H=2, T=700, seed=22, gate=gate, h0_std=0.3)
    o, hf = gpu_run(x)
    check(x, o, hf, TOL_BF16)


def test_matches_per_key_dim_forward_with_broadcast_gate():
    """gla_fwd_scalar equals gla_fwd given the same gate in every key dim."""
    say("[scalar vs broadcast] B=2 H=2 T=900")
    x = make_inputs(_wl("bf16", 128), B=2, H=2, T=900, seed=23, h0_std=0.2)
    o, hf = gpu_run(x)
    d = {n: x[n].to(DEV) for n in ("q", "k", "v", "h0")}
    gk = x["g"][..., None].expand(-1, -1, -1, 128).contiguous().to(DEV)
    o2, hf2 = gla.gla_fwd(d["q"], d["k"], d["v"], gk, d["h0"], want_final=True)
    torch.cuda.synchronize()
    eo = nerr(o, o2.float().cpu().numpy())
    eh = nerr(hf, hf2.cpu().numpy())
    say(f"    difference to gla_fwd: o {eo:.2e}, h_final {eh:.2e}")
    assert eo <= 1e-6 and eh <= 1e-6


def test_full_size_workload():
    """The benchmark's workload (prefill_16k_scalar) and launch configuration:
    every output element and final state against the oracle."""
    wl = SCALAR_WORKLOADS["prefill_16k_scalar"]
    say(f"[full {wl.name}] B={wl.B} H={wl.H} T={wl.T}, all {wl.B * wl.H} sequences")
    x = make_inputs(wl)
    o, hf = gpu_run(x, want_final=wl.want_final)
    check(x, o, hf, TOL_BF16)
