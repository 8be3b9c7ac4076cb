"""fp64 CPU definitions of the gated linear attention prefill forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything here is
plain, slow and written straight from the definitions on the pages:

* recurrence (blog "Linear Attention 在 GPU 上到底慢在哪", section 学长的反馈:
  the D x D state update h <- h*g + k^T v; "线性注意力GPU算子库的定义与技术解析",
  section 四, pseudocode: update the state, then read the output from it),
  with the gate as a log-decay on the key axis: S_t = diag(exp g_t) S_{t-1} +
  k_t^T v_t, o_t = scale * q_t S_t;
* the chunk form in words ("线性注意力GPU算子库的定义与技术解析", section 三.1 and
  section 四 GPU flow steps 1-3: split the sequence into chunks, pass states
  between chunks, compute the within-chunk output with matrix products).

Arrays are numpy float64 with layouts q,k,g [B,H,T,K], v [B,H,T,V],
h0 [B,H,K,V].
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_oracle_library(force: bool = True) -> str:
    """Compile ``gla_oracle.c`` with gcc (plain C, OpenMP) into liboracle.so."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def ensure_built() -> str:
    """Compile liboracle.so if it is missing.  Callers do this before anything
    touches the GPU: compiling starts gcc as a child process, which a process
    that has initialised the GPU must not do."""
    return build_oracle_library(force=False)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built: run __graft_entry__.build() or "
                               "oracle.reference.ensure_built() before any GPU work")
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gla_oracle_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                       ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                       ctypes.c_long, ctypes.c_long, ctypes.c_double,
                                       ctypes.c_long, ctypes.c_int]
        lib.gla_oracle_f64.restype = ctypes.c_int
        lib.gla_oracle_bwd_f64.argtypes = [dp] * 12 + [ctypes.c_long] * 5 + [
            ctypes.c_double, ctypes.c_long, ctypes.c_int]
        lib.gla_oracle_bwd_f64.restype = ctypes.c_int
        lib.gdn_oracle_f64.argtypes = [dp] * 8 + [ctypes.c_long] * 5 + [ctypes.c_double,
                                                                     ctypes.c_int]
        lib.gdn_oracle_f64.restype = ctypes.c_int
        lib.gla_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def oracle_threads() -> int:
    """Number of OpenMP threads the C oracle uses by default."""
    return int(_load().gla_oracle_max_threads())


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def token_recurrence(q, k, v, g, h0=None, scale=1.0, record_every=0, threads=0,
                     want_final=True):
    """The oracle: fp64 token-by-token recurrence (C, OpenMP).

    Returns ``(o, h_final, states)``; ``states`` (chunk-start states, the
    state before token n*record_every) is None unless ``record_every > 0``.
    """
    q, k, v, g, h0 = (_f64(x) for x in (q, k, v, g, h0))
    B, H, T, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, H, T, K) and g.shape == (B, H, T, K)
    assert v.shape == (B, H, T, V)
    if h0 is not None:
        assert h0.shape == (B, H, K, V)
    o = np.empty((B, H, T, V), dtype=np.float64)
    hf = np.empty((B, H, K, V), dtype=np.float64) if want_final else None
    states = None
    if record_every > 0:
        n = (T + record_every - 1) // record_every
        states = np.empty((B, H, n, K, V), dtype=np.float64)
    rc = _load().gla_oracle_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0),
                                _ptr(o), _ptr(hf), _ptr(states), B, H, T, K, V,
                                float(scale), int(record_every), int(threads))
    if rc != 0:
        raise RuntimeError(f"gla_oracle_f64 failed with status {rc}")
    return o, hf, states


def token_recurrence_backward(q, k, v, g, h0, do, dh_final, scale=1.0, threads=0, ckpt=64):
    """The oracle's backward (C, fp64): reverse-mode chain rule of the token
    recurrence, token by token (see gla_oracle.c).  ``h0`` and ``dh_final``
    may be None (zero).  Returns ``(dq, dk, dv, dg, dh0)``."""
    q, k, v, g, h0, do, dh_final = (_f64(x) for x in (q, k, v, g, h0, do, dh_final))
    B, H, T, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, H, T, K) and g.shape == (B, H, T, K)
    assert v.shape == (B, H, T, V) and do.shape == (B, H, T, V)
    for x in (h0, dh_final):
        if x is not None:
            assert x.shape == (B, H, K, V)
    dq = np.empty((B, H, T, K))
    dk = np.empty((B, H, T, K))
    dv = np.empty((B, H, T, V))
    dg = np.empty((B, H, T, K))
    dh0 = np.empty((B, H, K, V))
    rc = _load().gla_oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(do),
                                    _ptr(dh_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                    _ptr(dh0), B, H, T, K, V, float(scale), int(ckpt),
                                    int(threads))
    if rc != 0:
        raise RuntimeError(f"gla_oracle_bwd_f64 failed with status {rc}")
    return dq, dk, dv, dg, dh0


def brute_force(q, k, v, g, h0=None, scale=1.0):
    """O(T^2) evaluation of the unrolled recurrence, fp64.

    o_t = scale * [ (q_t * exp(G_t)) . h0 + sum_{s<=t} ((q_t * exp(G_t - G_s)) . k_s) v_s ]
    with G_t = sum_{r<=t} g_r (inclusive).  Unrolling S_t = diag(e^{g_t}) S_{t-1}
    + k_t^T v_t gives S_t = diag(e^{G_t}) h0 + sum_{s<=t} diag(e^{G_t-G_s}) k_s^T v_s.
    Also returns h_final = S_{T-1}.  Loops over t; tiny inputs only.
    """
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    B, H, T, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, H, T, V))
    hf = np.zeros((B, H, K, V))
    for b in range(B):
        for h in range(H):
            G = np.cumsum(g[b, h], axis=0)  # [T, K]
            base = np.zeros((K, V)) if h0 is None else np.asarray(h0[b, h], np.float64)
            for t in range(T):
                acc = (q[b, h, t] * np.exp(G[t])) @ base
                for s in range(t + 1):
                    w = np.dot(q[b, h, t] * np.exp(G[t] - G[s]), k[b, h, s])
                    acc = acc + w * v[b, h, s]
                o[b, h, t] = scale * acc
            if T > 0:
                S = np.exp(G[T - 1])[:, None] * base
                for s in range(T):
                    S = S + np.outer(k[b, h, s] * np.exp(G[T - 1] - G[s]), v[b, h, s])
                hf[b, h] = S
            else:
                hf[b, h] = base
    return o, hf


def closed_form_zero_gate(q, k, v, h0=None, scale=1.0):
    """g == 0 closed form: o = scale * [((Q K^T) * M) V + Q h0], h_final = h0 + K^T V.

    M is the lower-triangular causal mask including the diagonal.  Plain numpy
    matrix products per (b, h).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, H, T, V))
    hf = np.zeros((B, H, K, V))
    M = np.tril(np.ones((T, T)))
    for b in range(B):
        for h in range(H):
            Q, Kk, Vv = q[b, h], k[b, h], v[b, h]
            h0bh = np.zeros((K, V)) if h0 is None else np.asarray(h0[b, h], np.float64)
            o[b, h] = scale * (((Q @ Kk.T) * M) @ Vv + Q @ h0bh)
            hf[b, h] = h0bh + Kk.T @ Vv
    return o, hf


def chunk_cumsum(g, chunk):
    """Chunk-local inclusive cumsum of the log-gates (the 'cumsum' stage).

    Gc[n*C + i] = sum_{j<=i} g[n*C + j] (restarting at every chunk start) and
    Gamma[n] = Gc at the chunk's last valid row.  Returns (Gc [B,H,T,K],
    Gamma [B,H,N,K]).
    """
    g = np.asarray(g, dtype=np.float64)
    B, H, T, K = g.shape
    n = (T + chunk - 1) // chunk
    Gc = np.empty_like(g)
    Gam = np.empty((B, H, n, K))
    for c in range(n):
        lo, hi = c * chunk, min(T, (c + 1) * chunk)
        Gc[:, :, lo:hi] = np.cumsum(g[:, :, lo:hi], axis=2)
        Gam[:, :, c] = Gc[:, :, hi - 1]
    return Gc, Gam


def intra_scores(q, k, g, chunk, scale=1.0):
    """Within-chunk decayed causal scores, by definition.

    A[n, i, j] = scale * sum_d q[nC+i, d] k[nC+j, d] exp(Gc[nC+i, d] - Gc[nC+j, d])
    for j <= i, and 0 above the diagonal and outside the valid rows.  Returns
    [B, H, N, C, C]; the exponent is formed directly (no factorisation).
    """
    q, k = (np.asarray(x, dtype=np.float64) for x in (q, k))
    B, H, T, K = q.shape
    Gc, _ = chunk_cumsum(g, chunk)
    n = (T + chunk - 1) // chunk
    A = np.zeros((B, H, n, chunk, chunk))
    for c in range(n):
        lo, hi = c * chunk, min(T, (c + 1) * chunk)
        L = hi - lo
        qc, kc, Gcc = q[:, :, lo:hi], k[:, :, lo:hi], Gc[:, :, lo:hi]
        # E[b,h,i,j,d] = exp(Gc_i - Gc_j); only j <= i is kept
        diff = Gcc[:, :, :, None, :] - Gcc[:, :, None, :, :]
        mask = np.tril(np.ones((L, L), dtype=bool))
        diff = np.where(mask[None, None, :, :, None], diff, -np.inf)
        prod = qc[:, :, :, None, :] * kc[:, :, None, :, :] * np.exp(diff)
        A[:, :, c, :L, :L] = scale * prod.sum(axis=-1)
    return A


def chunked_reference(q, k, v, g, h0=None, scale=1.0, chunk=64):
    """The chunk form in fp64, as a second evaluation of the same sums.

    Per chunk n (rows i, j of the chunk, Gc and Gamma from ``chunk_cumsum``):
      o_i     = scale * [ (q_i * exp(Gc_i)) S_n + sum_{j<=i} A_ij v_j ]
      S_{n+1} = diag(exp(Gamma_n)) S_n + (k * exp(Gamma_n - Gc))^T V_n
    with A from the definition in ``intra_scores``.  Returns (o, h_final,
    chunk-start states [B,H,N,K,V]).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, T, K = q.shape
    V = v.shape[-1]
    Gc, Gam = chunk_cumsum(g, chunk)
    A = intra_scores(q, k, g, chunk, scale=1.0)
    n = (T + chunk - 1) // chunk
    o = np.zeros((B, H, T, V))
    states = np.zeros((B, H, n, K, V))
    hf = np.zeros((B, H, K, V))
    for b in range(B):
        for h in range(H):
            S = np.zeros((K, V)) if h0 is None else np.array(h0[b, h], dtype=np.float64)
            for c in range(n):
                lo, hi = c * chunk, min(T, (c + 1) * chunk)
                L = hi - lo
                states[b, h, c] = S
                Qh = q[b, h, lo:hi] * np.exp(Gc[b, h, lo:hi])
                o[b, h, lo:hi] = scale * (Qh @ S + A[b, h, c, :L, :L] @ v[b, h, lo:hi])
                Kh = k[b, h, lo:hi] * np.exp(Gam[b, h, c][None, :] - Gc[b, h, lo:hi])
                S = np.exp(Gam[b, h, c])[:, None] * S + Kh.T @ v[b, h, lo:hi]
            hf[b, h] = S
    return o, hf, states


# --- scalar-gate variant (one log-decay per token and head) -------------------
#
# The pages name Mamba-2's SSD / semiseparable block and Lightning Attention
# next to GLA (blog "Linear Attention 在 GPU 上到底慢在哪", section 正确的
# baseline 和下一步) but print no formula for them.  Reading taken here: the
# same recurrence with one gate per token shared by every key dim,
#     S_t = exp(g_t) S_{t-1} + k_t^T v_t,   o_t = scale * q_t S_t,
# g of shape [B,H,T].


def scalar_gate_recurrence(q, k, v, g, h0=None, scale=1.0, threads=0, want_final=True):
    """Scalar-gate recurrence via the token recurrence with g broadcast over
    the key dims (a per-token gate is the per-key-dim gate with equal
    entries).  g is [B,H,T]; returns (o, h_final)."""
    g = np.asarray(g, dtype=np.float64)
    K = np.shape(q)[-1]
    gk = np.ascontiguousarray(np.repeat(g[..., None], K, axis=-1))
    o, hf, _ = token_recurrence(q, k, v, gk, h0, scale, threads=threads, want_final=want_final)
    return o, hf


def scalar_gate_quadratic(q, k, v, g, h0=None, scale=1.0):
    """The masked quadratic (semiseparable-matrix) form of the scalar-gate
    recurrence, from unrolling it: with G_t = sum_{r<=t} g_r,
        o   = scale * [ ((Q K^T) * L) V + exp(G) * (Q h0) ],
        L_ts = exp(G_t - G_s) for s <= t, else 0,
        h_final = exp(G_{T-1}) h0 + sum_s exp(G_{T-1} - G_s) k_s^T v_s.
    Plain numpy matrix products per (b, h); O(T^2) memory, small T only."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    B, H, T, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, H, T, V))
    hf = np.zeros((B, H, K, V))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        for h in range(H):
            G = np.cumsum(g[b, h])
            L = np.where(causal, np.exp(np.where(causal, G[:, None] - G[None, :], 0.0)), 0.0)
            Q, Kk, Vv = q[b, h], k[b, h], v[b, h]
            base = np.zeros((K, V)) if h0 is None else np.asarray(h0[b, h], np.float64)
            o[b, h] = scale * (((Q @ Kk.T) * L) @ Vv + np.exp(G)[:, None] * (Q @ base))
            if T > 0:
                w = np.exp(G[T - 1] - G)
                hf[b, h] = np.exp(G[T - 1]) * base + (Kk * w[:, None]).T @ Vv
            else:
                hf[b, h] = base
    return o, hf


# --- gated delta rule (Gated DeltaNet forward) ---------------------------------
#
# The evaluation page ("面向长序列大模型的线性注意力算子性能评测方法与优化实践",
# sections 一 and 三.3) describes the GDN class only as gating plus an
# incremental ("delta") state update.  Reading taken: the published gated
# delta rule with a scalar gate and write strength per token and head,
#     S_t = exp(g_t) (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
#     o_t = scale q_t S_t.


def gdn_recurrence(q, k, v, g, beta, h0=None, scale=1.0, threads=0, want_final=True):
    """The oracle for the gated delta rule (C, fp64, token by token).

    q, k [B,H,T,K]; v [B,H,T,V]; g, beta [B,H,T]; h0 [B,H,K,V] or None.
    Returns (o, h_final)."""
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, H, T, K = q.shape
    V = v.shape[-1]
    assert k.shape == (B, H, T, K) and v.shape == (B, H, T, V)
    assert g.shape == (B, H, T) and beta.shape == (B, H, T)
    o = np.empty((B, H, T, V))
    hf = np.empty((B, H, K, V)) if want_final else None
    rc = _load().gdn_oracle_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                _ptr(o), _ptr(hf), B, H, T, K, V, float(scale), int(threads))
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_f64 failed with status {rc}")
    return o, hf


def gdn_chunked_reference(q, k, v, g, beta, h0=None, scale=1.0, chunk=64):
    """The gated delta rule in chunk form, fp64, as a second evaluation.

    Unrolling the recurrence inside a chunk from its start state S (gamma_i =
    exp of the chunk-local inclusive cumsum of g):
      the written rows u_i = beta_i (v_i - exp(g_i) k_i S_{i-1}) satisfy
      (I + A) U = diag(beta) V - diag(beta gamma) K S,
      A_ij = beta_i (gamma_i / gamma_j) (k_i . k_j) for j < i;
      o_i = scale [gamma_i q_i S + sum_{j<=i} (gamma_i / gamma_j) (q_i . k_j) u_j];
      S_next = gamma_last S + sum_j (gamma_last / gamma_j) k_j^T u_j.
    The triangular system is solved with numpy.linalg.solve."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, H, T, K = q.shape
    V = v.shape[-1]
    o = np.zeros((B, H, T, V))
    hf = np.zeros((B, H, K, V))
    for b in range(B):
        for h in range(H):
            S = np.zeros((K, V)) if h0 is None else np.array(h0[b, h], dtype=np.float64)
            for lo in range(0, T, chunk):
                hi = min(T, lo + chunk)
                n = hi - lo
                Q, Kc, Vc = q[b, h, lo:hi], k[b, h, lo:hi], v[b, h, lo:hi]
                bt = beta[b, h, lo:hi]
                G = np.cumsum(g[b, h, lo:hi])
                ratio = np.exp(G[:, None] - G[None, :])          # gamma_i / gamma_j
                strict = np.tril(np.ones((n, n)), -1)
                A = bt[:, None] * ratio * (Kc @ Kc.T) * strict
                rhs = bt[:, None] * Vc - (bt * np.exp(G))[:, None] * (Kc @ S)
                U = np.linalg.solve(np.eye(n) + A, rhs)
                P = (Q @ Kc.T) * ratio * np.tril(np.ones((n, n)))
                o[b, h, lo:hi] = scale * (np.exp(G)[:, None] * (Q @ S) + P @ U)
                S = np.exp(G[-1]) * S + (Kc * np.exp(G[-1] - G)[:, None]).T @ U
            hf[b, h] = S
    return o, hf
