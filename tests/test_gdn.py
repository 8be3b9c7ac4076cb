"""GPU parity of the gated delta rule forward (include/gla_gdn.h) against the
fp64 oracle (oracle.gdn_recurrence, token by token).

Bar: max|x - x_ref| / max|x_ref| <= 1e-2 for the bf16 output and for the
final state (bf16 operands in the matrix products, fp32 accumulation and
fp32 triangular solve), and no NaN/Inf.
"""

import sys

import numpy as np
import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import GDN_WORKLOADS, make_gdn_inputs
from wholecheck import select_f64, whole_errors

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def nerr(out, ref):
    out = np.asarray(out, dtype=np.float64)
    return float(np.max(np.abs(out - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


@pytest.fixture(autouse=True)
def _default_schedule():
    gla.set_tuning(0, 0)
    gla.gdn_set_path("auto")
    yield
    gla.set_tuning(0, 0)
    gla.gdn_set_path("auto")


def gpu_run(x, want_final=True):
    d = {n: (None if x[n] is None else x[n].to(DEV)) for n in ("q", "k", "v", "g", "beta", "h0")}
    o, hf = gla.gla_gdn_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], want_final=want_final)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (None if hf is None else hf.cpu().numpy())


def check(x, o, hf):
    """Every output element and final state against the oracle (in groups of
    sequences), normalised over the whole tensor."""
    B, H, T, K = x["q"].shape
    scale = K ** -0.5

    def ref(sel):
        f = select_f64(x, ("q", "k", "v", "g", "beta", "h0"), sel)
        ro, rh = oracle.gdn_recurrence(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"], scale)
        return {"o": ro, "h_final": rh}

    errs = whole_errors({"o": o, "h_final": hf}, ref, B, H, T)
    e, eh = errs["o"], errs.get("h_final")
    say(f"    o err {e:.3e}" + ("" if eh is None else f"  h_final err {eh:.3e}") + f"  (tol {TOL:g})")
    assert e <= TOL
    if eh is not None:
        assert eh <= TOL


BASE = GDN_WORKLOADS["gdn_b16_4k"]

SMALL = [
    # (B, H, T, D, h0)
    (1, 2, 1, 128, True),
    (2, 3, 63, 128, False),
    (2, 2, 65, 128, True),
    (1, 2, 300, 128, True),
    (2, 2, 1000, 128, False),
    (1, 2, 777, 64, True),
    (1, 3, 200, 64, False),
]


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("B,H,T,D,h0", SMALL)
def test_small_shapes(B, H, T, D, h0, path):
    say(f"[gdn {path}] B={B} H={H} T={T} D={D} h0={h0}")
    import dataclasses
    wl = dataclasses.replace(BASE, D=D)
    x = make_gdn_inputs(wl, B=B, H=H, T=T, seed=T + D + 5, h0_std=0.5 if h0 else None)
    gla.gdn_set_path(path)
    o, hf = gpu_run(x)
    check(x, o, hf)


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("gate,beta", [("const:-30", None), ("const:-10000", None), ("ls41", None),
                                       ("ls16", 1.0), ("ls16", 0.0), ("zero", 1.0)])
def test_extreme_gates_and_writes(gate, beta, path):
    say(f"[gdn extreme {path}] gate={gate} beta={beta}")
    x = make_gdn_inputs(BASE, B=1, H=2, T=500, seed=61, gate=gate, beta=beta, h0_std=0.3)
    gla.gdn_set_path(path)
    o, hf = gpu_run(x)
    check(x, o, hf)


@pytest.mark.parametrize("target", [1, 32, 0])
def test_value_block_split(target):
    """One-launch form: value columns split over 1, 2 (B*H = 16, target 32) or
    8 (default) work-groups per head give the same result."""
    say(f"[gdn value blocks] target_wgs={target}")
    x = make_gdn_inputs(BASE, B=2, H=8, T=333, seed=63, h0_std=0.2)
    gla.gdn_set_path("one")
    gla.set_tuning(target, 0)
    o, hf = gpu_run(x)
    check(x, o, hf)


@pytest.mark.parametrize("target", [1, 8, 0])
def test_value_block_split_d64(target):
    """The same at D = 64 (four waves): value columns over 1 (every wave owns
    columns, the one that solves T's diagonal blocks included), 2 or 4 (only the
    first waves own columns) work-groups per head."""
    import dataclasses
    say(f"[gdn value blocks D=64] target_wgs={target}")
    wl = dataclasses.replace(BASE, D=64)
    x = make_gdn_inputs(wl, B=2, H=2, T=333, seed=64, h0_std=0.2)
    gla.gdn_set_path("one")
    gla.set_tuning(target, 0)
    o, hf = gpu_run(x)
    check(x, o, hf)


@pytest.mark.parametrize("window,slices_target", [(1, 0), (3, 0), (2, 1), (0, 100000)])
def test_two_launch_windows_and_slices(window, slices_target):
    """Two-launch form over windows of 1 or 3 chunks (state carried between
    windows in the workspace, h0 given) and with 1 .. all prep slices; T
    leaves a ragged last chunk."""
    say(f"[gdn two windows] window={window} target={slices_target}")
    x = make_gdn_inputs(BASE, B=1, H=3, T=450, seed=64, h0_std=0.3)
    gla.gdn_set_path("two", window)
    gla.set_tuning(slices_target, 0)
    o, hf = gpu_run(x)
    check(x, o, hf)


def test_two_launch_matches_one_launch():
    """Both forms on the same inputs agree to bf16 rounding."""
    say("[gdn one vs two] B=2 H=4 T=1000")
    x = make_gdn_inputs(BASE, B=2, H=4, T=1000, seed=65, h0_std=0.2)
    gla.gdn_set_path("one")
    o1, h1 = gpu_run(x)
    gla.gdn_set_path("two")
    o2, h2 = gpu_run(x)
    eo, eh = nerr(o2, o1), nerr(h2, h1)
    say(f"    two vs one: o {eo:.2e}  h_final {eh:.2e}")
    assert eo <= 1e-2 and eh <= 1e-2
    check(x, o2, h2)


def test_zero_length_sequence():
    say("[gdn T=0]")
    q = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device=DEV)
    s = torch.empty(1, 2, 0, device=DEV)
    h0 = torch.randn(1, 2, 128, 128, device=DEV)
    o, hf = gla.gla_gdn_fwd(q, q, q, s, s, h0, want_final=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and torch.equal(hf, h0)


@pytest.mark.parametrize("path", ["one", "two"])
def test_bitwise_repeatable(path):
    say(f"[gdn repeatable {path}]")
    x = make_gdn_inputs(BASE, B=2, H=2, T=700, seed=62)
    gla.gdn_set_path(path)
    a = gpu_run(x)
    b = gpu_run(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["gdn_b16_4k", "gdn_16k"])
def test_full_size_workload(name):
    """The benchmark's workloads in its launch configuration (default schedule:
    one launch at B*H = 256, two launches at B*H = 16): every output element
    and final state against the oracle."""
    wl = GDN_WORKLOADS[name]
    say(f"[gdn full {name}] B={wl.B} H={wl.H} T={wl.T}, all {wl.B * wl.H} sequences")
    x = make_gdn_inputs(wl)
    o, hf = gpu_run(x)
    check(x, o, hf)
