"""ctypes binding of libgla.so (include/gla.h, include/gla_scalar.h,
include/gla_bwd.h, include/gla_gdn.h, include/gla_decode.h, include/gla_stages.h).

Argument marshalling only: shape/dtype/device checks, output allocation with
torch, and the call.  Every step of the computation runs in the HIP kernels
of libgla.so.  If the library has not been built, calls raise
``GLALibraryMissing``; there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgla.so")

GLA_OK = 0
ERRORS = {
    -1: "GLA_ERR_NULL", -2: "GLA_ERR_SHAPE", -3: "GLA_ERR_UNSUPPORTED", -4: "GLA_ERR_ALIGN",
    -5: "GLA_ERR_LAUNCH", -6: "GLA_ERR_ALLOC", -7: "GLA_ERR_ALIAS", -8: "GLA_ERR_DEVICE",
    -9: "GLA_ERR_WORKSPACE",
}

# every symbol include/gla.h and include/gla_stages.h declare
EXPORTED = ("gla_fwd", "gla_fwd_f32", "gla_set_tuning", "gla_strerror", "gla_version",
            "gla_release", "gla_profile_start", "gla_profile_stop", "gla_stage_cumsum",
            "gla_stage_intra", "gla_stage_states", "gla_decode", "gla_decode_f32",
            "gla_fwd_scalar", "gla_fwd_scalar_f32", "gla_bwd", "gla_bwd_f32", "gla_gdn_fwd",
            "gla_gdn_set_path", "gla_workspace_bytes", "gla_fwd_noalloc")
KERNEL_KINDS = {0: "output", 1: "segment", 2: "scan", 3: "other", 4: "decode", 5: "bwd_segment",
                6: "bwd", 7: "gdn", 8: "gdn_prep", 9: "gdn_walk",
                10: "states"}
GDN_PATHS = {"auto": 0, "one": 1, "two": 2}


class _KernelTime(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("ms", ctypes.c_float)]


class GLALibraryMissing(RuntimeError):
    pass


class GLAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgla.so and declare the C signatures (no GPU call is made)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise GLALibraryMissing(
            f"{path} is not built; run `python -m chunked_state_recurrence_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.gla_fwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.gla_fwd_f32.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.gla_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.gla_fwd_scalar.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.gla_bwd.argtypes = [P] * 12 + [I, I, I, I, I, I, F, P]
    lib.gla_bwd_f32.argtypes = [P] * 12 + [I, I, I, I, I, I, F, P]
    lib.gla_gdn_fwd.argtypes = [P] * 8 + [I, I, I, I, I, I, F, P]
    lib.gla_fwd_scalar_f32.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.gla_stage_states.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
    lib.gla_stage_cumsum.argtypes = [P, P, P, I, I, I, I, I, P]
    lib.gla_stage_intra.argtypes = [P, P, P, P, I, I, I, I, I, F, P]
    lib.gla_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, F, P]
    lib.gla_decode_f32.argtypes = [P, P, P, P, P, P, I, I, I, I, F, P]
    lib.gla_set_tuning.argtypes = [I, I]
    lib.gla_gdn_set_path.argtypes = [I, I]
    lib.gla_strerror.argtypes = [I]
    lib.gla_strerror.restype = ctypes.c_char_p
    lib.gla_version.argtypes = []
    lib.gla_release.argtypes = []
    lib.gla_workspace_bytes.argtypes = []
    lib.gla_workspace_bytes.restype = ctypes.c_longlong
    lib.gla_release.restype = None
    lib.gla_profile_start.argtypes = [I]
    lib.gla_profile_stop.argtypes = [ctypes.POINTER(_KernelTime), I, ctypes.POINTER(I)]
    lib.gla_profile_start.restype = ctypes.c_int
    lib.gla_profile_stop.restype = ctypes.c_int
    for name in ("gla_fwd", "gla_fwd_f32", "gla_fwd_noalloc", "gla_stage_states", "gla_stage_cumsum",
                 "gla_stage_intra", "gla_set_tuning", "gla_version", "gla_decode", "gla_decode_f32",
                 "gla_fwd_scalar", "gla_fwd_scalar_f32", "gla_bwd", "gla_bwd_f32", "gla_gdn_fwd",
                 "gla_gdn_set_path"):
        getattr(lib, name).restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(code: int):
    if code != GLA_OK:
        raise GLAError(code, load_library().gla_strerror(code).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _fwd(fn, io_dtype, q, k, v, g, h0, chunk, scale, want_final, o, h_final, stream,
         states=None, scalar_gate=False):
    B, H, T, K = q.shape
    V = v.shape[-1]
    dev = q.device
    gshape = (B, H, T) if scalar_gate else (B, H, T, K)
    for t, n, dt, shp in ((q, "q", io_dtype, (B, H, T, K)), (k, "k", io_dtype, (B, H, T, K)),
                          (v, "v", io_dtype, (B, H, T, V)), (g, "g", torch.float32, gshape),
                          (h0, "h0", torch.float32, (B, H, K, V))):
        _need(t, n, dt, shp, dev)
    if scale is None:
        scale = K ** -0.5
    if o is None:
        o = torch.empty((B, H, T, V), dtype=io_dtype, device=dev)
    _need(o, "o", io_dtype, (B, H, T, V), dev)
    if want_final and h_final is None:
        h_final = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    _need(h_final, "h_final", torch.float32, (B, H, K, V), dev)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(o), _ptr(h_final)]
    if states is not None:
        args.append(_ptr(states))
    rc = fn(*args, B, H, T, K, V, int(chunk), float(scale), _stream(stream))
    _check(rc)
    return o, h_final


def gla_fwd(q, k, v, g, h0=None, *, chunk=0, scale=None, want_final=False, o=None,
            h_final=None, stream=None):
    """bf16 forward: q, k, v bf16 [B,H,T,D]; g fp32 [B,H,T,D]; h0 fp32 [B,H,D,D] or None.

    Returns (o bf16 [B,H,T,D], h_final fp32 [B,H,D,D] or None).
    """
    return _fwd(load_library().gla_fwd, torch.bfloat16, q, k, v, g, h0, chunk, scale,
                want_final, o, h_final, stream)


def gla_fwd_noalloc(q, k, v, g, h0=None, *, chunk=0, scale=None, want_final=False, o=None,
                    h_final=None, stream=None):
    """gla_fwd through the entry point that allocates nothing on the device:
    its segment-state workspace is the library's static scratch (64 MiB per
    device).  Pass o (and h_final) to keep the call free of allocation; this
    wrapper otherwise allocates them with torch before the call."""
    return _fwd(load_library().gla_fwd_noalloc, torch.bfloat16, q, k, v, g, h0, chunk, scale,
                want_final, o, h_final, stream)


def gla_fwd_f32(q, k, v, g, h0=None, *, chunk=0, scale=None, want_final=False, o=None,
                h_final=None, stream=None):
    """fp32 forward: the same operation with fp32 q, k, v and o."""
    return _fwd(load_library().gla_fwd_f32, torch.float32, q, k, v, g, h0, chunk, scale,
                want_final, o, h_final, stream)


def gla_fwd_scalar(q, k, v, g, h0=None, *, chunk=0, scale=None, want_final=False, o=None,
                   h_final=None, stream=None):
    """Scalar-gate bf16 forward: as gla_fwd, with g fp32 [B,H,T] (one log-decay
    per token and head, shared by every key dim)."""
    return _fwd(load_library().gla_fwd_scalar, torch.bfloat16, q, k, v, g, h0, chunk, scale,
                want_final, o, h_final, stream, scalar_gate=True)


def gla_fwd_scalar_f32(q, k, v, g, h0=None, *, chunk=0, scale=None, want_final=False, o=None,
                       h_final=None, stream=None):
    """Scalar-gate fp32 forward: fp32 q, k, v, o; g fp32 [B,H,T]."""
    return _fwd(load_library().gla_fwd_scalar_f32, torch.float32, q, k, v, g, h0, chunk, scale,
                want_final, o, h_final, stream, scalar_gate=True)


def _bwd(fn, io_dtype, q, k, v, g, h0, do, dh_final, chunk, scale, want_dh0, out, stream):
    B, H, T, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if do is None:
        raise ValueError("do is required")
    for t, n, dt, shp in ((q, "q", io_dtype, (B, H, T, K)), (k, "k", io_dtype, (B, H, T, K)),
                          (v, "v", io_dtype, (B, H, T, V)), (g, "g", torch.float32, (B, H, T, K)),
                          (do, "do", io_dtype, (B, H, T, V)),
                          (h0, "h0", torch.float32, (B, H, K, V)),
                          (dh_final, "dh_final", torch.float32, (B, H, K, V))):
        _need(t, n, dt, shp, dev)
    if scale is None:
        scale = K ** -0.5
    out = dict(out or {})
    shapes = {"dq": ((B, H, T, K), io_dtype), "dk": ((B, H, T, K), io_dtype),
              "dv": ((B, H, T, V), io_dtype), "dg": ((B, H, T, K), torch.float32),
              "dh0": ((B, H, K, V), torch.float32)}
    for n, (shp, dt) in shapes.items():
        if out.get(n) is None and (n != "dh0" or want_dh0):
            out[n] = torch.empty(shp, dtype=dt, device=dev)
        _need(out.get(n), n, dt, shp, dev)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(do), _ptr(dh_final),
              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
              _ptr(out.get("dh0")), B, H, T, K, V, int(chunk), float(scale), _stream(stream)))
    return out["dq"], out["dk"], out["dv"], out["dg"], out.get("dh0")


def gla_bwd(q, k, v, g, h0, do, dh_final=None, *, chunk=0, scale=None, want_dh0=True, out=None,
            stream=None):
    """bf16 backward: returns (dq, dk, dv bf16; dg fp32 [B,H,T,K]; dh0 fp32 or None).
    ``out`` may hold preallocated dq, dk, dv, dg, dh0 tensors."""
    return _bwd(load_library().gla_bwd, torch.bfloat16, q, k, v, g, h0, do, dh_final, chunk,
                scale, want_dh0, out, stream)


def gla_bwd_f32(q, k, v, g, h0, do, dh_final=None, *, chunk=0, scale=None, want_dh0=True,
                out=None, stream=None):
    """fp32 backward: the same with fp32 q, k, v, do, dq, dk, dv."""
    return _bwd(load_library().gla_bwd_f32, torch.float32, q, k, v, g, h0, do, dh_final, chunk,
                scale, want_dh0, out, stream)


def gla_gdn_fwd(q, k, v, g, beta, h0=None, *, chunk=0, scale=None, want_final=False, o=None,
            h_final=None, stream=None):
    """Gated delta rule forward: q, k, v bf16 [B,H,T,D]; g, beta fp32 [B,H,T];
    h0 fp32 [B,H,D,D] or None.  Returns (o bf16, h_final fp32 or None)."""
    B, H, T, K = q.shape
    V = v.shape[-1]
    dev = q.device
    for t, n, dt, shp in ((q, "q", torch.bfloat16, (B, H, T, K)), (k, "k", torch.bfloat16, (B, H, T, K)),
                          (v, "v", torch.bfloat16, (B, H, T, V)), (g, "g", torch.float32, (B, H, T)),
                          (beta, "beta", torch.float32, (B, H, T)),
                          (h0, "h0", torch.float32, (B, H, K, V))):
        _need(t, n, dt, shp, dev)
    if scale is None:
        scale = K ** -0.5
    if o is None:
        o = torch.empty((B, H, T, V), dtype=torch.bfloat16, device=dev)
    _need(o, "o", torch.bfloat16, (B, H, T, V), dev)
    if want_final and h_final is None:
        h_final = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    _need(h_final, "h_final", torch.float32, (B, H, K, V), dev)
    _check(load_library().gla_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                  _ptr(h_final), B, H, T, K, V, int(chunk), float(scale),
                                  _stream(stream)))
    return o, h_final


def _decode(fn, io_dtype, q, k, v, g, state, scale, o, stream):
    B, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    for t, n, dt, shp in ((q, "q", io_dtype, (B, H, K)), (k, "k", io_dtype, (B, H, K)),
                          (v, "v", io_dtype, (B, H, V)), (g, "g", torch.float32, (B, H, K)),
                          (state, "state", torch.float32, (B, H, K, V))):
        if t is None:
            raise ValueError(f"{n} is required")
        _need(t, n, dt, shp, dev)
    if scale is None:
        scale = K ** -0.5
    if o is None:
        o = torch.empty((B, H, V), dtype=io_dtype, device=dev)
    _need(o, "o", io_dtype, (B, H, V), dev)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _ptr(o), B, H, K, V, float(scale),
              _stream(stream)))
    return o


def gla_decode(q, k, v, g, state, *, scale=None, o=None, stream=None):
    """One decode step, bf16: q, k bf16 [B,H,K], v bf16 [B,H,V], g fp32 [B,H,K];
    state fp32 [B,H,K,V] is updated in place.  Returns o bf16 [B,H,V]."""
    return _decode(load_library().gla_decode, torch.bfloat16, q, k, v, g, state, scale, o, stream)


def gla_decode_f32(q, k, v, g, state, *, scale=None, o=None, stream=None):
    """One decode step with fp32 q, k, v and o."""
    return _decode(load_library().gla_decode_f32, torch.float32, q, k, v, g, state, scale, o, stream)


def gla_stage_states(q, k, v, g, h0=None, *, chunk=64, scale=None, stream=None):
    """bf16 forward that also returns the chunk-start states [B,H,N,D,D] fp32."""
    B, H, T, K = q.shape
    n = (T + chunk - 1) // chunk
    states = torch.empty((B, H, n, K, v.shape[-1]), dtype=torch.float32, device=q.device)
    o, hf = _fwd(load_library().gla_stage_states, torch.bfloat16, q, k, v, g, h0, chunk, scale,
                 True, None, None, stream, states=states)
    return o, hf, states


def gla_stage_cumsum(g, *, chunk=64, stream=None):
    """Chunk-local cumsum of g: returns (Gc [B,H,T,D], Gamma [B,H,N,D]) fp32."""
    B, H, T, K = g.shape
    _need(g, "g", torch.float32, (B, H, T, K), g.device)
    n = (T + chunk - 1) // chunk
    gc = torch.empty_like(g)
    gam = torch.empty((B, H, n, K), dtype=torch.float32, device=g.device)
    _check(load_library().gla_stage_cumsum(_ptr(g), _ptr(gc), _ptr(gam), B, H, T, K, int(chunk),
                                           _stream(stream)))
    return gc, gam


def gla_stage_intra(q, k, g, *, chunk=64, scale=None, stream=None):
    """Scaled intra-chunk scores A [B,H,N,C,C] fp32 (bf16 q, k; fp32 g)."""
    B, H, T, K = q.shape
    for t, n, dt in ((q, "q", torch.bfloat16), (k, "k", torch.bfloat16), (g, "g", torch.float32)):
        _need(t, n, dt, (B, H, T, K), q.device)
    if scale is None:
        scale = K ** -0.5
    n = (T + chunk - 1) // chunk
    A = torch.empty((B, H, n, chunk, chunk), dtype=torch.float32, device=q.device)
    _check(load_library().gla_stage_intra(_ptr(q), _ptr(k), _ptr(g), _ptr(A), B, H, T, K,
                                          int(chunk), float(scale), _stream(stream)))
    return A


def set_tuning(target_wgs: int = 0, head_group: int = 0):
    _check(load_library().gla_set_tuning(int(target_wgs), int(head_group)))


def gdn_set_path(path: str = "auto", window_chunks: int = 0):
    """Form of gla_gdn_fwd: "auto", "one" (one launch) or "two" (prep + walk);
    window_chunks > 0 caps the two-launch windows (chunks of 64 tokens)."""
    _check(load_library().gla_gdn_set_path(GDN_PATHS[path], int(window_chunks)))


def profile_start(capacity: int):
    """Start tracing launches (HIP events around each kernel on its stream)."""
    _check(load_library().gla_profile_start(int(capacity)))


def profile_stop():
    """Stop tracing; returns [(kind_name, ms), ...] in launch order."""
    lib = load_library()
    buf = (_KernelTime * 65536)()
    n = ctypes.c_int(0)
    _check(lib.gla_profile_stop(buf, 65536, ctypes.byref(n)))
    return [(KERNEL_KINDS.get(buf[i].kind, "other"), float(buf[i].ms)) for i in range(n.value)]


def version() -> int:
    return int(load_library().gla_version())


def strerror(code: int) -> str:
    return load_library().gla_strerror(int(code)).decode()


def release():
    load_library().gla_release()


def workspace_bytes() -> int:
    """Device workspace the library holds on the current device (bytes)."""
    return int(load_library().gla_workspace_bytes())
