"""Whole-tensor comparison with the fp64 oracle, in groups of (batch, head)
sequences.

Every output element and every final state is compared; the oracle runs over
a bounded number of token-heads at a time so that the float64 copies of a
full-size workload (up to 2M token-heads) stay a few hundred MiB.  The
normalised error is taken over the whole tensor: max over all elements of
|x - x_ref| divided by max over all elements of |x_ref| (the bar of the
evaluation page "面向长序列大模型的线性注意力算子性能评测方法与优化实践", section
六.1, against a high-precision token-by-token reference).
"""

from __future__ import annotations

import numpy as np
import torch


def head_groups(B: int, H: int, T: int, token_heads: int = 1 << 18):
    """(b, h) pairs in groups of at most ``token_heads`` token-heads (at least one pair)."""
    per = max(1, token_heads // max(T, 1))
    pairs = [(b, h) for b in range(B) for h in range(H)]
    return [pairs[i:i + per] for i in range(0, len(pairs), per)]


def select_f64(x: dict, names, sel):
    """The sequences ``sel`` of each CPU tensor in ``x`` as float64 numpy
    arrays of shape [1, len(sel), ...] (None stays None)."""
    out = {}
    for n in names:
        t = x.get(n)
        out[n] = None if t is None else (
            torch.stack([t[b, h] for (b, h) in sel])[None].to(torch.float64).numpy())
    return out


def take(a: np.ndarray, sel):
    return np.stack([a[b, h] for (b, h) in sel])[None]


def whole_errors(got: dict, ref_fn, B: int, H: int, T: int, token_heads: int = 1 << 18):
    """Normalised errors over whole tensors.

    ``got`` maps a name to the GPU result as a numpy array [B, H, ...] (None:
    not compared); ``ref_fn(sel)`` returns a dict with the oracle's arrays
    [1, len(sel), ...] for the same names.  Every array of ``got`` is checked
    finite.  Returns {name: max|x - x_ref| / max|x_ref|}.
    """
    num, den = {}, {}
    for n, a in got.items():
        if a is not None:
            assert np.isfinite(a).all(), f"non-finite {n}"
    for sel in head_groups(B, H, T, token_heads):
        ref = ref_fn(sel)
        for n, a in got.items():
            if a is None:
                continue
            r = ref[n]
            g = take(a, sel).astype(np.float64)
            num[n] = max(num.get(n, 0.0), float(np.max(np.abs(g - r))) if r.size else 0.0)
            den[n] = max(den.get(n, 0.0), float(np.max(np.abs(r))) if r.size else 0.0)
    return {n: num[n] / max(den[n], 1e-30) for n in num}
