"""CPU oracle for the gated linear attention prefill forward and its backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP library and never imports it.

Parity status of each function (what pins it is in ``tests/test_oracle.py``):

* ``token_recurrence`` (C, fp64): pinned by brute force, the g == 0 closed
  form, hand-derived golden fixtures, split invariance, the T == 1 and
  vanishing-gate special cases, and linearity / permutation invariants.
* ``brute_force``, ``closed_form_zero_gate``: pinned against each other, the
  golden fixtures and ``token_recurrence``.
* ``chunk_cumsum``: pinned by its definition against ``numpy.cumsum`` of the
  whole sequence and by the chunk totals.
* ``intra_scores``: pinned against ``brute_force`` (the within-chunk part of
  the output) and against a direct O(C^2 K) loop on tiny inputs.
* ``chunked_reference``: pinned against ``token_recurrence`` at several chunk
  sizes (chunking is a reordering of the same sums).
* ``token_recurrence_backward`` (C, fp64): the reverse-mode chain rule of the
  same recurrence; pinned against torch autograd through an independent
  PyTorch forward, central finite differences, hand-derived golden fixtures
  (``tests/golden/backward/``) and the identity that dg is the reverse cumsum
  of q*dq - k*dk plus the final-state term.
* ``gdn_recurrence`` (C, fp64: the gated delta rule token by token) and
  ``gdn_chunked_reference`` (its chunk form with a triangular solve): pinned
  against each other at several chunk sizes, a hand-derived fixture
  (``tests/golden/gdn/``), the beta = 0 closed form (pure decay of h0), the
  exact-overwrite behaviour for orthonormal keys with beta = 1, and split
  invariance.
* ``scalar_gate_recurrence`` (scalar gate g [B,H,T], through
  ``token_recurrence``) and ``scalar_gate_quadratic`` (the masked quadratic
  form): pinned against each other, a hand-derived golden fixture
  (``tests/golden/scalar/``), the g == 0 closed form and the T == 1 case.
"""

from .reference import (  # noqa: F401
    brute_force,
    build_oracle_library,
    chunk_cumsum,
    chunked_reference,
    closed_form_zero_gate,
    gdn_chunked_reference,
    gdn_recurrence,
    intra_scores,
    oracle_threads,
    scalar_gate_quadratic,
    scalar_gate_recurrence,
    token_recurrence,
    token_recurrence_backward,
)
