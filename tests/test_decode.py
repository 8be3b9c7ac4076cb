"""GPU parity of the decode step (include/gla_decode.h) against the fp64 oracle.

A decode step is the recurrence of the prefill path for one token: the
oracle is the same token-by-token recurrence (oracle.token_recurrence), run
over T = 1 from the carried state, or over the whole sequence when several
steps are chained.  Bar: the normalised error of the prefill tests
(max|x - x_ref| / max|x_ref|), 1e-2 for bf16 output, 1e-3 for fp32 output;
the fp32 state is held to 1e-4 in both (it is updated with fp32 FMAs from
exactly the inputs the oracle sees, so only fp32 rounding separates them).
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import WORKLOADS, make_inputs, to_f64_numpy

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 1e-2, "f32": 1e-3}
TOL_STATE = 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def nerr(out, ref):
    out = np.asarray(out, dtype=np.float64)
    return float(np.max(np.abs(out - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def _wl(dtype, D):
    base = WORKLOADS["tiny_f32"] if dtype == "f32" else WORKLOADS["prefill_4k"]
    return dataclasses.replace(base, D=D, dtype=dtype)


def _inputs(dtype, D, B, H, T, gate="ls16", seed=11, h0_std=0.5):
    return make_inputs(_wl(dtype, D), B=B, H=H, T=T, gate=gate, seed=seed, h0_std=h0_std)


def _step_fn(dtype):
    return gla.gla_decode if dtype == "bf16" else gla.gla_decode_f32


def _decode_steps(x, dtype, steps, state):
    """Run `steps` decode calls over tokens 0..steps-1 of x; returns o [B,H,steps,V]."""
    d = {n: x[n].to(DEV) for n in ("q", "k", "v", "g")}
    scale = d["q"].shape[-1] ** -0.5
    outs = []
    for t in range(steps):
        o = _step_fn(dtype)(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                            d["v"][:, :, t].contiguous(), d["g"][:, :, t].contiguous(), state,
                            scale=scale)
        outs.append(o)
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2).float().cpu().numpy()


def _oracle(x, T, h0):
    f = {n: to_f64_numpy(x[n][:, :, :T]) for n in ("q", "k", "v", "g")}
    scale = f["q"].shape[-1] ** -0.5
    o, hf, _ = oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], to_f64_numpy(h0), scale)
    return o, hf


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("gate", ["ls16", "ls41", "zero", "const:-1e4"])
def test_single_step(dtype, D, gate):
    say(f"decode single step dtype={dtype} D={D} gate={gate}")
    x = _inputs(dtype, D, B=3, H=5, T=1, gate=gate)
    state = x["h0"].to(DEV).clone()
    o = _decode_steps(x, dtype, 1, state)
    ro, rh = _oracle(x, 1, x["h0"])
    e, es = nerr(o, ro), nerr(state.cpu().numpy(), rh)
    say(f"    o err {e:.3e}  state err {es:.3e}")
    assert np.isfinite(o).all()
    assert e <= TOL[dtype] and es <= TOL_STATE


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_chained_steps_from_zero_state(dtype, D):
    """96 decode steps from a zero state equal the recurrence over 96 tokens."""
    say(f"decode chained dtype={dtype} D={D}")
    x = _inputs(dtype, D, B=2, H=3, T=96, gate="ls41", seed=12, h0_std=None)
    B, H = 2, 3
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device=DEV)
    o = _decode_steps(x, dtype, 96, state)
    ro, rh = _oracle(x, 96, None)
    e, es = nerr(o, ro), nerr(state.cpu().numpy(), rh)
    say(f"    o err {e:.3e}  state err {es:.3e}")
    assert e <= TOL[dtype] and es <= TOL_STATE


@pytest.mark.parametrize("T0", [1, 300])
def test_prefill_then_decode(T0):
    """gla_fwd over T0 tokens hands its final state to 20 decode steps; the
    outputs of both equal the recurrence over T0 + 20 tokens."""
    say(f"prefill {T0} then decode 20")
    D, B, H, T1 = 128, 2, 4, 20
    x = _inputs("bf16", D, B=B, H=H, T=T0 + T1, seed=13, h0_std=0.1)
    d = {n: x[n].to(DEV) for n in ("q", "k", "v", "g", "h0")}
    pre = {n: d[n][:, :, :T0].contiguous() for n in ("q", "k", "v", "g")}
    o_pre, state = gla.gla_fwd(pre["q"], pre["k"], pre["v"], pre["g"], d["h0"], want_final=True)
    rest = {n: x[n][:, :, T0:].contiguous() for n in ("q", "k", "v", "g")}
    o_dec = _decode_steps(rest, "bf16", T1, state)
    o = np.concatenate([o_pre.float().cpu().numpy(), o_dec], axis=2)
    ro, rh = _oracle(x, T0 + T1, x["h0"])
    e, es = nerr(o, ro), nerr(state.cpu().numpy(), rh)
    say(f"    o err {e:.3e}  state err {es:.3e}")
    assert e <= TOL["bf16"] and es <= TOL["bf16"]


def test_many_rows():
    """1024 (batch, head) rows in one call (a decode batch of 64 x 16 heads)."""
    say("decode 64 x 16 rows")
    D, B, H = 128, 64, 16
    x = _inputs("bf16", D, B=B, H=H, T=1, seed=14, h0_std=0.3)
    state = x["h0"].to(DEV).clone()
    o = _decode_steps(x, "bf16", 1, state)
    ro, rh = _oracle(x, 1, x["h0"])
    e, es = nerr(o, ro), nerr(state.cpu().numpy(), rh)
    say(f"    o err {e:.3e}  state err {es:.3e}")
    assert e <= TOL["bf16"] and es <= TOL_STATE


def test_output_buffer_and_stream():
    """A caller-given o, written on a side stream."""
    say("decode into a given buffer on a side stream")
    D, B, H = 64, 2, 2
    x = _inputs("f32", D, B=B, H=H, T=1, seed=15)
    d = {n: x[n][:, :, 0].contiguous().to(DEV) for n in ("q", "k", "v", "g")}
    state = x["h0"].to(DEV).clone()
    o = torch.full((B, H, D), 7.0, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gla.gla_decode_f32(d["q"], d["k"], d["v"], d["g"], state, o=o, scale=0.25, stream=s)
    s.synchronize()
    f = {n: to_f64_numpy(x[n]) for n in ("q", "k", "v", "g")}
    ro, rh, _ = oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], to_f64_numpy(x["h0"]), 0.25)
    assert nerr(o.cpu().numpy(), ro[:, :, 0]) <= TOL["f32"]
    assert nerr(state.cpu().numpy(), rh) <= TOL_STATE


def test_full_size_decode_workload():
    """The benchmark's decode workload (256 sequences x 16 heads, D = 128) in
    its launch configuration: one step over every row, every output and every
    updated state against the oracle."""
    from chunked_state_recurrence_amd.workloads import DECODE_WORKLOADS
    wl = DECODE_WORKLOADS["decode_b256"]
    say(f"[decode full {wl.name}] B={wl.B} H={wl.H} D={wl.D}, all {wl.B * wl.H} rows")
    x = make_inputs(wl)
    d = {n: x[n][:, :, 0].contiguous().to(DEV) for n in ("q", "k", "v", "g")}
    state = x["h0"].to(DEV).clone()
    o = gla.gla_decode(d["q"], d["k"], d["v"], d["g"], state, scale=wl.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    st = state.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(st).all()
    f = {n: to_f64_numpy(x[n][:, :, :1]) for n in ("q", "k", "v", "g")}
    ro, rh, _ = oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], to_f64_numpy(x["h0"]),
                                        wl.scale)
    e, es = nerr(o[:, :, None], ro), nerr(st, rh)
    say(f"    o err {e:.3e}  state err {es:.3e}")
    assert e <= TOL["bf16"] and es <= TOL_STATE
