"""The library's cached device workspace (include/gla.h: gla_workspace_bytes,
gla_release).

A forward call with several segments per head holds the segment states:
(B*H) * (segments - 1) * K * (V + 1) * 4 bytes at the default schedule; a
backward call adds its chunk-start states.  gla_release frees all of it, and
the next call allocates it again and returns the same result bitwise.
"""

import sys

import pytest
import torch

import chunked_state_recurrence_amd as gla

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_release_and_regrow():
    gla.set_tuning(0, 0)
    B, H, T, D = 1, 4, 1000, 128   # 16 chunks of 64: one chunk per segment, 16 segments per head
    gen = torch.Generator().manual_seed(11)
    q, k, v, do = (torch.randn(B, H, T, D, generator=gen).bfloat16().to(DEV) for _ in range(4))
    g = (torch.nn.functional.logsigmoid(torch.randn(B, H, T, D, generator=gen)) / 16).to(DEV)

    _say("[workspace] release")
    torch.cuda.synchronize()
    gla.release()
    assert gla.workspace_bytes() == 0

    _say("[workspace] forward")
    o1, h1 = gla.gla_fwd(q, k, v, g, None, want_final=True)
    torch.cuda.synchronize()
    fwd_bytes = gla.workspace_bytes()
    assert fwd_bytes >= B * H * (16 - 1) * D * (D + 1) * 4

    _say("[workspace] backward")
    gla.gla_bwd(q, k, v, g, None, do)
    torch.cuda.synchronize()
    # the chunk-start states (bf16 at D = 128, chunk 64) come on top
    assert gla.workspace_bytes() >= fwd_bytes + B * H * 16 * D * D * 2

    _say("[workspace] release, then the forward again")
    gla.release()
    assert gla.workspace_bytes() == 0
    o2, h2 = gla.gla_fwd(q, k, v, g, None, want_final=True)
    torch.cuda.synchronize()
    assert gla.workspace_bytes() >= B * H * (16 - 1) * D * (D + 1) * 4
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    gla.release()
    assert gla.workspace_bytes() == 0
