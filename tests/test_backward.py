"""GPU parity of the backward (include/gla_bwd.h) against the fp64 oracle
(oracle.token_recurrence_backward, the chain rule of the token recurrence).

Bar, per gradient (dq, dk, dv, dg, dh0): max|x - x_ref| / max|x_ref| <= 1e-2
for the bf16 path (bf16 operands in the matrix products, as in the forward),
<= 1e-3 for the fp32 path, and no NaN/Inf.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import WORKLOADS, make_grad_inputs, make_inputs
from wholecheck import select_f64, whole_errors

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_F32 = 1e-3
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dg", "dh0")


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
    return dataclasses.replace(base, D=D)


def gpu_bwd(x, gr, *, fp32=False, chunk=0):
    d = {n: (None if x[n] is None else x[n].to(DEV)) for n in ("q", "k", "v", "g", "h0")}
    do = gr["do"].to(DEV)
    dhf = None if gr["dh_final"] is None else gr["dh_final"].to(DEV)
    fn = gla.gla_bwd_f32 if fp32 else gla.gla_bwd
    out = fn(d["q"], d["k"], d["v"], d["g"], d["h0"], do, dhf, chunk=chunk)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in out]


def check(x, gr, got, tol):
    """Every gradient element against the oracle (in groups of sequences),
    normalised over each whole tensor."""
    src = dict(x)
    src["do"], src["dhf"] = gr["do"], gr["dh_final"]
    B, H, T, K = x["q"].shape
    scale = K ** -0.5

    def ref(sel):
        f = select_f64(src, ("q", "k", "v", "g", "h0", "do", "dhf"), sel)
        r = oracle.token_recurrence_backward(f["q"], f["k"], f["v"], f["g"], f["h0"], f["do"],
                                             f["dhf"], scale)
        return dict(zip(NAMES, r))

    errs = whole_errors(dict(zip(NAMES, got)), ref, B, H, T)
    say("    " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()) + f"  (tol {tol:g})")
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad


@pytest.mark.parametrize("gate", ["ls16", "zero"])
@pytest.mark.parametrize("chunk", [64, 32])
def test_f32_tiny(gate, chunk):
    say(f"[bwd f32] D=64 T=256 gate={gate} chunk={chunk}")
    wl = _wl("f32", 64)
    x = make_inputs(wl, gate=gate, h0_std=0.5)
    gr = make_grad_inputs(wl, T=256)
    check(x, gr, gpu_bwd(x, gr, fp32=True, chunk=chunk), TOL_F32)


@pytest.mark.parametrize("chunk", [32, 0])   # 0: the backward's default (32 at this shape)
def test_f32_head_dim_128(chunk):
    say(f"[bwd f32] D=128 T=200 chunk={chunk}")
    wl = _wl("f32", 128)
    x = make_inputs(wl, T=200, H=2, h0_std=0.3)
    gr = make_grad_inputs(wl, T=200, H=2)
    check(x, gr, gpu_bwd(x, gr, fp32=True, chunk=chunk), TOL_F32)


SMALL = [
    # (B, H, T, D, chunk, h0, dh_final)
    (1, 2, 1, 128, 64, True, True),
    (2, 3, 63, 128, 64, False, True),
    (2, 2, 65, 128, 64, True, False),
    (1, 3, 200, 128, 32, True, True),
    (2, 2, 1000, 128, 64, True, True),
    (1, 2, 777, 64, 64, True, True),
    (1, 2, 300, 64, 32, False, False),
]


@pytest.mark.parametrize("B,H,T,D,chunk,h0,dhf", SMALL)
def test_bf16_small_shapes(B, H, T, D, chunk, h0, dhf):
    say(f"[bwd bf16] B={B} H={H} T={T} D={D} chunk={chunk} h0={h0} dh_final={dhf}")
    wl = _wl("bf16", D)
    x = make_inputs(wl, B=B, H=H, T=T, seed=T + D + 2, h0_std=0.5 if h0 else None)
    gr = make_grad_inputs(wl, B=B, H=H, T=T, seed=T + D, dh_final=dhf)
    check(x, gr, gpu_bwd(x, gr, chunk=chunk), TOL_BF16)


@pytest.mark.parametrize("target", [1, 4, 64])
def test_bf16_segment_splits(target):
    """1 .. N segments: the backward segment pass and its scan are exercised."""
    say(f"[bwd segments] target_wgs={target}")
    wl = _wl("bf16", 128)
    x = make_inputs(wl, B=1, H=2, T=1000, seed=31, h0_std=0.3)
    gr = make_grad_inputs(wl, B=1, H=2, T=1000, seed=31)
    gla.set_tuning(target, 0)
    check(x, gr, gpu_bwd(x, gr), TOL_BF16)


@pytest.mark.parametrize("T", [576, 1100, 1343])
def test_bf16_segment_unit_lengths(T):
    """Segments of 3, 6 and 7 chunks (three per head): every remainder after
    the segment pass's rounds of four chunks."""
    say(f"[bwd segment lengths] T={T}")
    wl = _wl("bf16", 128)
    x = make_inputs(wl, B=1, H=2, T=T, seed=T + 7, h0_std=0.3)
    gr = make_grad_inputs(wl, B=1, H=2, T=T, seed=T + 7)
    gla.set_tuning(6, 0)
    check(x, gr, gpu_bwd(x, gr), TOL_BF16)


@pytest.mark.parametrize("gate", ["const:-30", "const:-10000", "ls41", "mixed"])
def test_bf16_extreme_gates(gate):
    """Chunks past the span guard take the exact elementwise path."""
    say(f"[bwd extreme gates] {gate}")
    wl = _wl("bf16", 128)
    if gate == "mixed":
        x = make_inputs(wl, B=1, H=2, T=300, seed=32, h0_std=0.3)
        gen = torch.Generator().manual_seed(33)
        spikes = torch.rand(x["g"].shape, generator=gen) < 0.01
        x["g"] = torch.where(spikes, torch.full_like(x["g"], -200.0), x["g"])
    else:
        x = make_inputs(wl, B=1, H=2, T=300, seed=32, gate=gate, h0_std=0.3)
    gr = make_grad_inputs(wl, B=1, H=2, T=300, seed=32)
    check(x, gr, gpu_bwd(x, gr), TOL_BF16)


def test_zero_length_sequence():
    """T = 0: dh0 = dh_final."""
    say("[bwd T=0]")
    q = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device=DEV)
    g = torch.empty(1, 2, 0, 128, device=DEV)
    dhf = torch.randn(1, 2, 128, 128, device=DEV)
    dq, dk, dv, dg, dh0 = gla.gla_bwd(q, q, q, g, None, q, dhf)
    torch.cuda.synchronize()
    assert dq.shape == (1, 2, 0, 128) and torch.equal(dh0, dhf)


def test_bitwise_repeatable():
    say("[bwd repeatable]")
    wl = _wl("bf16", 128)
    x = make_inputs(wl, B=1, H=4, T=700, seed=34, h0_std=0.2)
    gr = make_grad_inputs(wl, B=1, H=4, T=700, seed=34)
    a = gpu_bwd(x, gr)
    b = gpu_bwd(x, gr)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_full_size_workload():
    """The benchmark's workload (prefill_16k) in its launch configuration:
    every gradient element of every head against the oracle."""
    wl = WORKLOADS["prefill_16k"]
    say(f"[bwd full {wl.name}] B={wl.B} H={wl.H} T={wl.T}, all {wl.B * wl.H} sequences")
    x = make_inputs(wl)
    gr = make_grad_inputs(wl)
    check(x, gr, gpu_bwd(x, gr), TOL_BF16)
