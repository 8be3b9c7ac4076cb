"""C-ABI checks that need no GPU: the library loads, exports every symbol the
headers declare, and rejects bad arguments with the documented codes before
anything is enqueued (fake device pointers are never dereferenced)."""

import ctypes
import glob
import os
import re

import pytest

import chunked_state_recurrence_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

pytestmark = pytest.mark.skipif(not os.path.exists(gla.LIB_PATH),
                                reason="libgla.so not built (run __graft_entry__.build())")


def _declared():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?(?:\w+\s+)*\w+\s*\*?\s*(gla_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_headers_declare_the_binding_symbols():
    assert sorted(gla.EXPORTED) == _declared()


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gla.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_host_only_calls():
    assert gla.version() == 100
    assert gla.strerror(0) == "ok"
    for code in range(-9, 0):
        assert gla.strerror(code) != "unknown error code"
    assert gla.strerror(-99) == "unknown error code"
    gla.set_tuning(0, 0)
    with pytest.raises(gla.GLAError):
        gla.set_tuning(-1, 0)


FAKE = 1 << 40          # 16-byte aligned, never dereferenced
STEP = 1 << 32          # far apart: no overlap between fake buffers


def _call(lib, fn="gla_fwd", **kw):
    a = dict(q=FAKE, k=FAKE + STEP, v=FAKE + 2 * STEP, g=FAKE + 3 * STEP, h0=None,
             o=FAKE + 4 * STEP, hf=None, B=1, H=2, T=100, K=128, V=128, chunk=64, scale=0.1)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return getattr(lib, fn)(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["h0"]),
                            vp(a["o"]), vp(a["hf"]), a["B"], a["H"], a["T"], a["K"], a["V"],
                            a["chunk"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(H=-1), -2), (dict(T=-5), -2), (dict(T=1 << 24), -2),
    (dict(K=128, V=64), -3), (dict(K=96, V=96), -3), (dict(chunk=48), -3), (dict(chunk=256), -3),
    (dict(q=None), -1), (dict(g=None), -1), (dict(o=None), -1),
    (dict(q=FAKE + 8), -4), (dict(hf=FAKE + 5 * STEP + 4), -4),
    (dict(o=FAKE + 64), -7), (dict(hf=FAKE + 4 * STEP + 4096), -7),
    (dict(h0=FAKE + 6 * STEP, hf=FAKE + 6 * STEP), -7),
])
@pytest.mark.parametrize("fn", ["gla_fwd", "gla_fwd_noalloc"])
def test_argument_errors(kw, code, fn):
    lib = gla.load_library()
    assert _call(lib, fn, **kw) == code


def test_noalloc_rejects_a_schedule_past_its_scratch():
    """gla_fwd_noalloc: a schedule whose segment states exceed the 64 MiB
    static scratch is refused before any device call (here 16 heads of 16K
    tokens split into 256 segments each: 255 x 16 states of 66 KB, 269 MB)."""
    lib = gla.load_library()
    gla.set_tuning(100000, 0)
    try:
        assert _call(lib, "gla_fwd_noalloc", H=16, T=16384) == -9
    finally:
        gla.set_tuning(0, 0)


# Scalar-gate entry points: g is [B,H,T] (800 bytes at B=1, H=2, T=100), so an
# output that starts inside those bytes is an alias.  (Cases that would pass
# validation are not called: fake pointers must never reach a launch.)
@pytest.mark.parametrize("fn", ["gla_fwd_scalar", "gla_fwd_scalar_f32"])
@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(T=1 << 24), -2), (dict(K=96, V=96), -3), (dict(chunk=48), -3),
    (dict(g=None), -1), (dict(q=None), -1), (dict(g=FAKE + 3 * STEP + 4), -4),
    (dict(o=FAKE + 3 * STEP + 784), -7), (dict(hf=FAKE + 3 * STEP + 512), -7),
])
def test_scalar_gate_argument_errors(fn, kw, code):
    lib = gla.load_library()
    assert _call(lib, fn, **{"chunk": 32, **kw}) == code   # chunk 32: valid for both dtypes


def _decode(lib, f32=False, **kw):
    a = dict(q=FAKE, k=FAKE + STEP, v=FAKE + 2 * STEP, g=FAKE + 3 * STEP, state=FAKE + 4 * STEP,
             o=FAKE + 5 * STEP, B=2, H=3, K=128, V=128, scale=0.1)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    fn = lib.gla_decode_f32 if f32 else lib.gla_decode
    return fn(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["state"]), vp(a["o"]),
              a["B"], a["H"], a["K"], a["V"], a["scale"], None)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(H=-1), -2), (dict(K=0, V=0), -2), (dict(B=1 << 16, H=1 << 15), -2),
    (dict(K=128, V=64), -3), (dict(K=32, V=32), -3), (dict(K=256, V=256), -3),
    (dict(q=None), -1), (dict(g=None), -1), (dict(state=None), -1), (dict(o=None), -1),
    (dict(v=FAKE + 2 * STEP + 8), -4), (dict(state=FAKE + 4 * STEP + 4), -4),
    (dict(o=FAKE + 64), -7),                      # o overlaps q
    (dict(state=FAKE + 3 * STEP + 16), -7),       # state overlaps g
    (dict(o=FAKE + 4 * STEP + 4096), -7),         # o inside state
])
def test_decode_argument_errors(kw, code, f32):
    lib = gla.load_library()
    assert _decode(lib, f32, **kw) == code


def _bwd(lib, fn="gla_bwd", **kw):
    a = dict(q=FAKE, k=FAKE + STEP, v=FAKE + 2 * STEP, g=FAKE + 3 * STEP, h0=None,
             do=FAKE + 4 * STEP, dhf=None, dq=FAKE + 5 * STEP, dk=FAKE + 6 * STEP,
             dv=FAKE + 7 * STEP, dg=FAKE + 8 * STEP, dh0=None,
             B=1, H=2, T=100, K=128, V=128, chunk=32, scale=0.1)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return getattr(lib, fn)(*(vp(a[n]) for n in ("q", "k", "v", "g", "h0", "do", "dhf", "dq", "dk",
                                                   "dv", "dg", "dh0")),
                            a["B"], a["H"], a["T"], a["K"], a["V"], a["chunk"], a["scale"], None)


@pytest.mark.parametrize("fn", ["gla_bwd", "gla_bwd_f32"])
@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(T=-1), -2), (dict(K=96, V=96), -3), (dict(chunk=48), -3),
    (dict(do=None), -1), (dict(dq=None), -1), (dict(dg=None), -1), (dict(g=None), -1),
    (dict(dk=FAKE + 6 * STEP + 8), -4), (dict(dh0=FAKE + 9 * STEP + 4), -4),
    (dict(dq=FAKE + 64), -7),                    # dq overlaps q
    (dict(dv=FAKE + 4 * STEP + 32), -7),         # dv overlaps do
    (dict(dk=FAKE + 5 * STEP + 64), -7),         # dk overlaps dq
    (dict(dh0=FAKE + 8 * STEP + 64), -7),        # dh0 overlaps dg
])
def test_backward_argument_errors(fn, kw, code):
    lib = gla.load_library()
    assert _bwd(lib, fn, **kw) == code


def test_backward_chunk_table():
    """The backward runs chunks 32 and 64 (fp32 at K = 128: 32 only); a chunk the
    forward also takes (128, or fp32 64 at K = 128) is rejected before any work."""
    lib = gla.load_library()
    assert _bwd(lib, "gla_bwd", chunk=128) == -3
    assert _bwd(lib, "gla_bwd", chunk=128, K=64, V=64) == -3
    assert _bwd(lib, "gla_bwd_f32", chunk=64) == -3              # K = 128
    assert _bwd(lib, "gla_bwd_f32", chunk=128, K=64, V=64) == -3


def _gdn(lib, **kw):
    a = dict(q=FAKE, k=FAKE + STEP, v=FAKE + 2 * STEP, g=FAKE + 3 * STEP, beta=FAKE + 4 * STEP,
             h0=None, o=FAKE + 5 * STEP, hf=None, B=1, H=2, T=100, K=128, V=128, chunk=0, scale=0.1)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.gla_gdn_fwd(*(vp(a[n]) for n in ("q", "k", "v", "g", "beta", "h0", "o", "hf")),
                       a["B"], a["H"], a["T"], a["K"], a["V"], a["chunk"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(T=-1), -2), (dict(K=128, V=64), -3), (dict(K=96, V=96), -3),
    (dict(chunk=32), -3), (dict(beta=None), -1), (dict(g=None), -1), (dict(o=None), -1),
    (dict(q=FAKE + 8), -4), (dict(o=FAKE + 64), -7), (dict(o=FAKE + 4 * STEP + 256), -7),
    (dict(hf=FAKE + 5 * STEP + 512), -7),
])
def test_gdn_argument_errors(kw, code):
    lib = gla.load_library()
    assert _gdn(lib, **kw) == code


def test_gdn_set_path_arguments():
    lib = gla.load_library()
    assert lib.gla_gdn_set_path(3, 0) == -2
    assert lib.gla_gdn_set_path(-1, 0) == -2
    assert lib.gla_gdn_set_path(2, -1) == -2
    for path in (1, 2, 0):
        assert lib.gla_gdn_set_path(path, 5) == 0
    assert lib.gla_gdn_set_path(0, 0) == 0


def test_fp32_chunk_support_table():
    lib = gla.load_library()
    vp = ctypes.c_void_p

    def f32(K, chunk):
        return lib.gla_fwd_f32(vp(FAKE), vp(FAKE + STEP), vp(FAKE + 2 * STEP), vp(FAKE + 3 * STEP),
                               None, vp(FAKE + 4 * STEP), None, 1, 1, 10, K, K, chunk, 1.0, None)
    # fp32 runs chunks of 32 and 64 tokens at both head dims; 128 is bf16 only
    assert f32(128, 128) == -3
    assert f32(64, 128) == -3
    assert f32(128, 96) == -3


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(gla.GLALibraryMissing):
        gla.load_library(str(tmp_path / "libgla.so"))


# Stage entry points: shapes are checked first, so fake pointers never reach
# a launch; T * K past 2^29 would overflow the kernels' 32-bit row offsets.
@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(H=-1), -2), (dict(T=-1), -2), (dict(T=1 << 24), -2),
    (dict(B=1 << 16, H=1 << 15), -2), (dict(K=96), -3), (dict(chunk=48), -3),
])
@pytest.mark.parametrize("stage", ["cumsum", "intra", "states"])
def test_stage_argument_errors(stage, kw, code):
    lib = gla.load_library()
    a = dict(B=1, H=2, T=100, K=128, chunk=64)
    a.update(kw)
    p = [ctypes.c_void_p(FAKE + i * STEP) for i in range(8)]
    if stage == "cumsum":
        r = lib.gla_stage_cumsum(p[0], p[1], p[2], a["B"], a["H"], a["T"], a["K"], a["chunk"], None)
    elif stage == "intra":
        r = lib.gla_stage_intra(p[0], p[1], p[2], p[3], a["B"], a["H"], a["T"], a["K"], a["chunk"],
                                ctypes.c_float(1.0), None)
    else:
        r = lib.gla_stage_states(p[0], p[1], p[2], p[3], None, p[4], None, p[5], a["B"], a["H"],
                                 a["T"], a["K"], a["K"], a["chunk"], ctypes.c_float(1.0), None)
    assert r == code
