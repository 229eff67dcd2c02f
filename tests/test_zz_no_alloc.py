"""txl_relattn_fwd_noalloc, the forward entry point that allocates nothing
(its key-split workspace is the library's static device scratch), against
txl_relattn_fwd with a caller workspace: bitwise-equal out and lse on two
calls in a row, the second smaller (the scratch keeps the first call's
partial outputs, which the second must fully overwrite), both within the
bf16 tolerance of the oracle; a call needing more than the scratch is refused
and writes nothing."""
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_xl_relative_rel_amd as txl
from transformer_xl_relative_rel_amd import synth

from tests._common import check_close, sharp_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(d):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(dt)
    return [t(d[x], torch.bfloat16) for x in ("q", "k", "v", "r")] + [t(d[x], torch.float32) for x in ("u", "vb")]


@pytest.mark.parametrize("first,second", [
    ((1, 16, 128, 1600, 0), (1, 8, 64, 300, 0)),     # streaming kernel's key splits, then a smaller call
    ((2, 8, 300, 256, 0), (1, 4, 160, 77, 3)),       # throughput kernel with key splits and the combine
])
def test_noalloc_matches_workspace_call(first, second):
    for B, H, L, M, splits in (first, second):
        log(f"case: noalloc B{B} H{H} L{L} M{M} splits{splits}")
        d = sharp_inputs(B, H, L, M, 0.5, seed=1400 + L + M)
        q, k, v, r, u, vb = _dev(d)
        assert txl.relattn_workspace_size(q, k, splits=splits) > 0, "the case must use the scratch"
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        txl.relattn_fwd_noalloc(q, k, v, r, u, vb, out, lse, splits=splits)
        ref, rlse = txl.relattn_fwd(q, k, v, r, u, vb, want_lse=True, splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), rlse.view(torch.int32))
        want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=16)
        check_close(out.float().cpu().numpy().astype(np.float64), want, "bf16", "noalloc out")
        assert np.abs(lse.cpu().numpy() - wlse).max() <= 2e-2


def test_noalloc_refuses_more_than_the_scratch():
    B, H, L, M, dh = 8, 16, 512, 512, 64
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16")
    q, k, v, r, u, vb = _dev(d)
    assert txl.relattn_workspace_size(q, k, splits=4) > (32 << 20)
    out = torch.zeros_like(q)
    with pytest.raises(txl.TxlError, match="scratch"):
        txl.relattn_fwd_noalloc(q, k, v, r, u, vb, out, splits=4)
    torch.cuda.synchronize()
    assert not out.any()
