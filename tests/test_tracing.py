"""Launch tracing (gla_profile_start / gla_profile_stop, include/gla.h).

The CPU test pins the binding's kind names to the GLA_KERNEL_* values the
header defines.  The GPU test checks, for one call of each entry point, the
launches the library records and their order: the forward's state pass, scan
and output pass; the backward's forward state pass, scan, states-only pass,
its own segment pass, scan and chunk pass; a decode step; the T = 0 copy of
h0 into h_final; that tracing stops at the capacity it was given; and the
gated delta rule's automatic form on each side of its boundary (prep + walk
while B*H*D/16 <= 256, one launch beyond).
"""

import re
import sys
from pathlib import Path

import pytest
import torch

import chunked_state_recurrence_amd as gla
from chunked_state_recurrence_amd import _binding

ROOT = Path(__file__).resolve().parents[1]
DEV = "cuda:0"


def test_kind_names_match_header():
    text = (ROOT / "include" / "gla.h").read_text()
    defined = {int(v): n.lower() for n, v in re.findall(r"#define\s+GLA_KERNEL_(\w+)\s+(\d+)", text)}
    assert defined, "no GLA_KERNEL_* values in include/gla.h"
    assert defined == _binding.KERNEL_KINDS


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _trace(fn, capacity=64):
    gla.profile_start(capacity)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        recs = gla.profile_stop()
    return recs


@pytest.mark.gpu
def test_launch_kinds_per_entry_point():
    gla.set_tuning(0, 0)
    B, H, T, D = 1, 4, 1000, 128   # 16 chunks of 64 per head: several segments per head
    gen = torch.Generator().manual_seed(7)
    q, k, v, do = (torch.randn(B, H, T, D, generator=gen).bfloat16().to(DEV) for _ in range(4))
    g = (torch.nn.functional.logsigmoid(torch.randn(B, H, T, D, generator=gen)) / 16).to(DEV)

    _say("[trace] forward")
    recs = _trace(lambda: gla.gla_fwd(q, k, v, g, None, want_final=True))
    assert [kind for kind, _ in recs] == ["segment", "scan", "output"]
    assert all(ms > 0 for _, ms in recs)

    _say("[trace] backward")
    recs = _trace(lambda: gla.gla_bwd(q, k, v, g, None, do))
    assert [kind for kind, _ in recs] == ["segment", "scan", "states", "bwd_segment", "scan", "bwd"]
    assert all(ms > 0 for _, ms in recs)

    _say("[trace] decode")
    st = torch.zeros(B, H, D, D, device=DEV)
    q1, k1, v1, g1 = (x[:, :, 0].contiguous() for x in (q, k, v, g))
    recs = _trace(lambda: gla.gla_decode(q1, k1, v1, g1, st))
    assert [kind for kind, _ in recs] == ["decode"]

    _say("[trace] T = 0")
    e = torch.empty(B, H, 0, D, device=DEV).bfloat16()
    h0 = torch.randn(B, H, D, D, generator=gen).to(DEV)
    recs = _trace(lambda: gla.gla_fwd(e, e, e, torch.empty(B, H, 0, D, device=DEV), h0, want_final=True))
    assert [kind for kind, _ in recs] == ["other"]

    _say("[trace] capacity")
    recs = _trace(lambda: gla.gla_fwd(q, k, v, g, None, want_final=True), capacity=2)
    assert [kind for kind, _ in recs] == ["segment", "scan"]


@pytest.mark.gpu
@pytest.mark.parametrize("D,BH,two", [(128, 32, True), (128, 40, False), (64, 64, True), (64, 72, False)])
def test_gdn_automatic_form(D, BH, two):
    # two launches (prep + walk) while the walk's B*H*D/16 one-wave work-groups
    # fit the 256 work-group target, one launch beyond (include/gla_gdn.h)
    gla.set_tuning(0, 0)
    gla.gdn_set_path("auto")
    B, H, T = BH // 8, 8, 128
    gen = torch.Generator().manual_seed(BH)
    q, k = (torch.nn.functional.normalize(torch.randn(B, H, T, D, generator=gen), dim=-1).bfloat16().to(DEV)
            for _ in range(2))
    v = torch.randn(B, H, T, D, generator=gen).bfloat16().to(DEV)
    g = (torch.nn.functional.logsigmoid(torch.randn(B, H, T, generator=gen)) / 16).to(DEV)
    beta = torch.sigmoid(torch.randn(B, H, T, generator=gen)).to(DEV)
    _say(f"[trace gdn auto] D={D} B*H={BH}")
    recs = _trace(lambda: gla.gla_gdn_fwd(q, k, v, g, beta, None))
    assert [kind for kind, _ in recs] == (["gdn_prep", "gdn_walk"] if two else ["gdn"])
