"""Parity of the HIP relative-attention backward (through the C ABI) with the
CPU oracle's backward (chain rule on the forward definition of [SRC]
RelPartialLearnableMultiHeadAttn.forward), plus properties fixed by the
mathematics.

The device path: txl_relattn_fwd gives out and lse, txl_relattn_bwd the
gradients (bf16 dq, dk, dv; fp32 dr, du, dvb).  The oracle takes the same
bf16-rounded q, k, v, r, the fp32 u, vb and the bf16 dout, in fp64.

Tolerance.  Every gradient is a sum over (query, key) pairs of a product of
two factors; on the device one factor (p or dS) is rounded to bf16 (unit
roundoff u = 2^-9) before the MFMA, the other is an exact bf16 input or a
query operand rounded once like the forward's, and the result is rounded once
more (dq, dk, dv to bf16).  p itself comes from logits with the forward's
rounding, and D_i from the bf16 output.  So each element is off by a few u
times the sum of its terms' magnitudes; sums of mixed-sign terms make that a
small multiple of the largest gradient of the tensor.  Bound:
max |err| <= 2e-2 * max |ref| and mean |err| <= 1e-2 * mean |ref| per tensor.
A wrong index or a dropped term moves whole rows by O(|ref|) and fails both.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_xl_relative_rel_amd as txl
from transformer_xl_relative_rel_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dr", "du", "dvb")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def inputs(B, H, L, M, std, seed=synth.SEED):
    d = synth.relattn_inputs(B, H, L, M, 64, dtype="bf16", std=std, seed=seed)
    d["dout"] = synth.round_bf16(synth.normal((B, H, L, 64), synth.STREAM["dout"], 1.0, seed).astype(np.float32))
    return d


def run_gpu(d, window=0, mem_valid=None):
    q, k, v, r, dout = (dev(d[x], torch.bfloat16) for x in ("q", "k", "v", "r", "dout"))
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    mv = None if mem_valid is None else torch.tensor(mem_valid, dtype=torch.int32, device=DEV)
    out, lse = txl.relattn_fwd(q, k, v, r, u, vb, want_lse=True, window=window, mem_valid=mv)
    # workspace filled with 0xff bytes (bf16 and fp32 NaN): a read of anything the
    # kernels did not write first shows up as a non-finite gradient
    nbytes = txl.relattn_bwd_workspace_size(q, k, v, r, out, dout, window=window, mem_valid=mv)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    grads = txl.relattn_bwd(q, k, v, r, u, vb, out, lse, dout, window=window, mem_valid=mv, workspace=ws)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in zip(NAMES, grads)}


def check(got, want, what, tol_max=2e-2, tol_mean=1e-2):
    for n in NAMES:
        g, w = got[n], want[n]
        assert g.shape == w.shape, (what, n, g.shape, w.shape)
        assert np.all(np.isfinite(g)), f"{what} {n}: non-finite"
        err = np.abs(g - w)
        ref_max, ref_mean = float(np.abs(w).max()), float(np.abs(w).mean())
        log(f"  {what} {n}: max err {err.max():.3e} (ref max {ref_max:.3e}), mean err {err.mean():.3e} "
            f"(ref mean {ref_mean:.3e})")
        assert err.max() <= tol_max * ref_max + 1e-6, f"{what} {n}: max err {err.max():.3e} vs ref max {ref_max:.3e}"
        assert err.mean() <= tol_mean * ref_mean + 1e-7, f"{what} {n}: mean err {err.mean():.3e} vs {ref_mean:.3e}"


CASES = [
    # B, H, L, M, std, window, mem_valid
    (1, 1, 1, 0, 1.0, 0, None),
    (1, 2, 16, 16, 1.0, 0, None),
    (2, 2, 40, 24, 0.5, 0, None),
    (1, 1, 7, 150, 1.0, 0, None),
    (2, 1, 130, 70, 0.5, 0, None),
    (1, 2, 64, 0, 1.0, 0, None),
    (1, 1, 200, 300, 0.25, 0, None),
    (2, 3, 129, 1, 0.5, 0, None),
    (1, 2, 256, 256, 0.125, 0, None),
    (2, 2, 40, 24, 0.5, 30, None),
    (2, 2, 40, 24, 0.5, 0, [5, 24]),
    (2, 1, 130, 70, 0.5, 50, [0, 33]),
    (9, 2, 40, 30, 0.5, 0, None),          # batch rows not a multiple of the dr kernel's 4 batch groups
    (2, 2, 64, 300, 0.5, 0, [20, 300]),    # row 0 hides keys 0..279: whole 128-key blocks never stored
    (1, 2, 70, 260, 0.5, 90, [3]),         # window and hidden blocks together
]


@pytest.mark.parametrize("B,H,L,M,std,window,mem_valid", CASES)
def test_bwd_matches_oracle(B, H, L, M, std, window, mem_valid):
    log(f"case: bwd B{B} H{H} L{L} M{M} std{std} window{window} mem_valid{mem_valid}")
    d = inputs(B, H, L, M, std)
    got = run_gpu(d, window, mem_valid)
    want = oracle.relattn_bwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], d["dout"], threads=8,
                              same_length=window, mem_valid=mem_valid)
    check(got, want, f"B{B} H{H} L{L} M{M}")


def test_bwd_single_key_closed_form():
    """L = 1, M = 0: one visible key, p = 1, so out = v, dS = 0 and every
    gradient but dv vanishes; dv = dout."""
    log("case: bwd single key")
    d = inputs(2, 3, 1, 0, 1.0)
    got = run_gpu(d)
    for n in ("dq", "dk", "dr", "du", "dvb"):
        assert np.abs(got[n]).max() <= 1e-6, n
    np.testing.assert_array_equal(got["dv"], d["dout"].astype(np.float64))


def test_bwd_hidden_memory_rows_get_zero():
    """Keys hidden by the per-row memory validity carry exactly zero dk, dv."""
    log("case: bwd hidden memory rows")
    d = inputs(2, 2, 48, 40, 0.5)
    got = run_gpu(d, mem_valid=[7, 40])
    assert not np.any(got["dk"][0, :, :33]) and not np.any(got["dv"][0, :, :33])


def test_bwd_is_deterministic_full_size():
    """Two backward calls at the benchmark shape give bitwise-equal results."""
    log("case: bwd determinism B8 H16 L512 M512")
    d = synth.relattn_inputs(8, 16, 512, 512, 64, dtype="bf16")
    dout = dev(synth.round_bf16(synth.normal((8, 16, 512, 64), synth.STREAM["dout"], 1.0).astype(np.float32)),
               torch.bfloat16)
    q, k, v, r = (dev(d[x], torch.bfloat16) for x in ("q", "k", "v", "r"))
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    out, lse = txl.relattn_fwd(q, k, v, r, u, vb, want_lse=True)
    a = txl.relattn_bwd(q, k, v, r, u, vb, out, lse, dout)
    b = txl.relattn_bwd(q, k, v, r, u, vb, out, lse, dout)
    torch.cuda.synchronize()
    for x, y, n in zip(a, b, NAMES):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), n


@pytest.mark.parametrize("B,H,L,M,std", [(8, 16, 512, 512, None), (8, 16, 512, 256, None), (1, 16, 128, 1600, None),
                                         (8, 16, 512, 512, 0.5)])
def test_bwd_full_size_every_head(B, H, L, M, std):
    """Benchmark shapes: the whole backward on the device against the oracle's
    backward of the whole call, every element of all six gradients (all
    heads and batch rows), at the configs' input scale and with sharp inputs
    (std 0.5, u and vb 0.5)."""
    log(f"case: bwd full size B{B} H{H} L{L} M{M} std {std}")
    if std is None:
        d = synth.relattn_inputs(B, H, L, M, 64, dtype="bf16")
    else:
        d = synth.relattn_inputs(B, H, L, M, 64, dtype="bf16", std=std, bias_std=0.5, seed=1301)
    d["dout"] = synth.round_bf16(synth.normal((B, H, L, 64), synth.STREAM["dout"], 1.0).astype(np.float32))
    got = run_gpu(d)
    want = oracle.relattn_bwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], d["dout"], threads=16)
    check(got, want, f"B{B} H{H} L{L} M{M}")


def test_bwd_strided_views_of_fused_qkv():
    """q, k, v as head views of one fused [B, K, 3, H, dh] projection buffer and
    out / dout in the merged-heads layout [B, L, H, dh] (the layout a decoder
    layer hands over); gradients come back with the same strides."""
    B, H, L, M = 2, 3, 70, 50
    K = M + L
    log(f"case: bwd strided B{B} H{H} L{L} M{M}")
    d = inputs(B, H, L, M, 0.5)
    qkv = torch.zeros((B, K, 3, H, 64), dtype=torch.bfloat16, device=DEV)
    qkv[:, M:, 0] = dev(d["q"], torch.bfloat16).permute(0, 2, 1, 3)
    qkv[:, :, 1] = dev(d["k"], torch.bfloat16).permute(0, 2, 1, 3)
    qkv[:, :, 2] = dev(d["v"], torch.bfloat16).permute(0, 2, 1, 3)
    q = qkv[:, M:, 0].permute(0, 2, 1, 3)
    k = qkv[:, :, 1].permute(0, 2, 1, 3)
    v = qkv[:, :, 2].permute(0, 2, 1, 3)
    r = dev(d["r"], torch.bfloat16)
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    out_m = torch.empty((B, L, H, 64), dtype=torch.bfloat16, device=DEV)
    out = out_m.permute(0, 2, 1, 3)
    _, lse = txl.relattn_fwd(q, k, v, r, u, vb, out=out, want_lse=True)
    dout_m = dev(d["dout"], torch.bfloat16).permute(0, 2, 1, 3).contiguous()
    dout = dout_m.permute(0, 2, 1, 3)
    grads = txl.relattn_bwd(q, k, v, r, u, vb, out, lse, dout)
    torch.cuda.synchronize()
    assert grads[0].stride() == q.stride() and grads[1].stride() == k.stride()
    got = {n: t.float().cpu().numpy().astype(np.float64) for n, t in zip(NAMES, grads)}
    want = oracle.relattn_bwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], d["dout"], threads=8)
    check(got, want, "strided")
