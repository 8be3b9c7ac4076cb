"""GPU test of gla_fwd_noalloc (include/gla.h), the forward entry point for
callers that cannot allocate device memory.

It runs the same kernels and schedule as gla_fwd with its segment-state
workspace in the library's static scratch, so on the same inputs its output
and final state must equal gla_fwd's bitwise; both are also compared with the
fp64 oracle to the forward's bar (max|x - x_ref| / max|x_ref| <= 1e-2 for
bf16 output and the final state).  Two calls in a row: the full prefill_16k
shape (B=1, H=16, T=16K, with h0), then a smaller input (B=2, H=3, T=1000),
so the second call runs on scratch contents the first one left; a third
call takes 128-token chunks (whose state pass runs on 64-token chunks, a
different schedule for the same scratch).  The
entry point is called through the C ABI with preallocated outputs; neither
the library's own workspace nor torch's allocations may change across it.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import chunked_state_recurrence_amd as gla
import oracle
from chunked_state_recurrence_amd.workloads import WORKLOADS, make_inputs
from wholecheck import select_f64, whole_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _abi_call(fn, d, o, hf, scale, chunk=0):
    B, H, T, K = d["q"].shape
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["h0"]), p(o), p(hf),
              B, H, T, K, K, chunk, ctypes.c_float(scale), stream)


def _oracle_errors(x, scale, o, hf):
    B, H, T = x["q"].shape[:3]

    def ref(sel):
        f = select_f64(x, ("q", "k", "v", "g", "h0"), sel)
        ro, rh, _ = oracle.token_recurrence(f["q"], f["k"], f["v"], f["g"], f["h0"], scale)
        return {"o": ro, "h_final": rh}

    return whole_errors({"o": o, "h_final": hf}, ref, B, H, T)


@pytest.mark.parametrize("case", [(1, 16, 16384, 0.02, 2, 0), (2, 3, 1000, 0.3, 7, 0), (1, 4, 3000, 0.1, 9, 128)],
                         ids=["prefill_16k_shape", "smaller_after", "chunk128_after"])
def test_noalloc_matches_gla_fwd(case):
    B, H, T, h0_std, seed, chunk = case
    wl = WORKLOADS["prefill_16k"]
    say(f"[noalloc] B={B} H={H} T={T} h0_std={h0_std} chunk={chunk}")
    lib = gla.load_library()
    gla.set_tuning(0, 0)
    x = make_inputs(wl, B=B, H=H, T=T, seed=seed, h0_std=h0_std)
    d = {n: x[n].to(DEV) for n in ("q", "k", "v", "g", "h0")}
    o_a = torch.empty(B, H, T, wl.D, dtype=torch.bfloat16, device=DEV)
    h_a = torch.empty(B, H, wl.D, wl.D, dtype=torch.float32, device=DEV)
    o_b, h_b = torch.empty_like(o_a), torch.empty_like(h_a)
    torch.cuda.synchronize()
    ws_before = gla.workspace_bytes()
    torch_before = torch.cuda.memory_allocated(DEV)
    rc = _abi_call(lib.gla_fwd_noalloc, d, o_a, h_a, wl.scale, chunk)
    torch.cuda.synchronize()
    assert rc == 0, gla.strerror(rc)
    assert gla.workspace_bytes() == ws_before, "gla_fwd_noalloc grew the library workspace"
    assert torch.cuda.memory_allocated(DEV) == torch_before
    assert _abi_call(lib.gla_fwd, d, o_b, h_b, wl.scale, chunk) == 0
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b), "output differs from gla_fwd"
    assert torch.equal(h_a, h_b), "final state differs from gla_fwd"
    errs = _oracle_errors(x, wl.scale, o_a.float().cpu().numpy(), h_a.cpu().numpy())
    say(f"    vs oracle: o {errs['o']:.3e}  h_final {errs['h_final']:.3e} (tol {TOL:g})")
    assert errs["o"] <= TOL and errs["h_final"] <= TOL
    assert np.isfinite(o_a.float().cpu().numpy()).all()
