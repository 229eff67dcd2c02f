"""Parity of the streaming path (short segments against a long memory: bf16,
dh = 64, L <= 128, no lower key bounds; one workgroup per key split with one
wave per 32-query run, splits merged by the split combine) with the CPU
oracle.  This is the
evaluation regime of the pages: a few new tokens per step attending over a
long cached memory ([XL] "Segment-Level Recurrence", evaluation with a longer
memory than in training).

Tolerances as for the other bf16 cases: max |err| <= 2e-2, mean |err| <=
2e-3 and <= 2% of the output RMS, lse within 2e-2."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_xl_relative_rel_amd as txl
from transformer_xl_relative_rel_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(d, **kw):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(dt)
    q, k, v, r = (t(d[x], torch.bfloat16) for x in ("q", "k", "v", "r"))
    u, vb = t(d["u"], torch.float32), t(d["vb"], torch.float32)
    out, lse = txl.relattn_fwd(q, k, v, r, u, vb, want_lse=True, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(got, glse, want, wlse, what):
    err = np.abs(got - want)
    rms = math.sqrt(float(np.mean(want ** 2)))
    assert err.max() <= 2e-2, f"{what} max err {err.max():.3e}"
    assert err.mean() <= 2e-3, f"{what} mean err {err.mean():.3e}"
    assert err.mean() <= 0.02 * rms, f"{what} mean err {err.mean():.3e} vs rms {rms:.3e}"
    assert np.abs(glse - wlse).max() <= 2e-2, f"{what} lse"


@pytest.mark.parametrize("B,H,L,M,splits", [
    (1, 4, 1, 1600, 0), (2, 4, 16, 1600, 0), (1, 4, 32, 1600, 0), (1, 4, 45, 1600, 0),
    (1, 2, 33, 700, 1), (1, 2, 33, 700, 3), (2, 2, 128, 1000, 5), (1, 2, 7, 0, 0), (1, 2, 100, 64, 2),
])
def test_stream_parity(B, H, L, M, splits):
    log(f"case: stream B{B} H{H} L{L} M{M} splits{splits}")
    d = synth.relattn_inputs(B, H, L, M, 64, dtype="bf16", seed=3333 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    got, glse = run_gpu(d, splits=splits)
    check(got, glse, want, wlse, f"L{L} M{M} splits{splits}")


@pytest.mark.parametrize("B,H,L,M,std,splits", [
    (1, 4, 1, 1600, 0.5, 0), (1, 4, 20, 1600, 0.8, 0), (2, 4, 45, 700, 0.5, 0), (1, 8, 77, 300, 0.7, 2),
    (1, 4, 100, 64, 0.5, 1), (1, 8, 128, 1600, 0.5, 0), (1, 2, 128, 0, 1.0, 1),
])
def test_stream_sharp_inputs(B, H, L, M, std, splits):
    """Inputs at std 0.5-1.0 (u, vb 0.5), on which a shifted or missing
    position term falls outside the tolerance: one to four runs per
    workgroup, ragged last runs, forced and automatic key splits."""
    log(f"case: stream sharp B{B} H{H} L{L} M{M} std{std} splits{splits}")
    d = synth.relattn_inputs(B, H, L, M, 64, dtype="bf16", std=std, bias_std=0.5, seed=5100 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    got, glse = run_gpu(d, splits=splits)
    check(got, glse, want, wlse, f"sharp L{L} M{M} splits{splits}")


def test_stream_deterministic():
    log("case: stream determinism")
    d = synth.relattn_inputs(1, 8, 24, 1600, 64, dtype="bf16", seed=4)
    a, la = run_gpu(d)
    b, lb = run_gpu(d)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
