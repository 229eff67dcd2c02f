"""Parity of the HIP relative-attention kernel (through the C ABI) with the CPU
oracle, plus probes whose answers are fixed by the method itself.

Tolerances (tests/_common.py): fp32 path max |err| <= 1e-4; bf16 path (bf16
inputs, fp32 accumulation, bf16 output) against the fp64 oracle on the same
bf16 inputs: max |err| <= 2e-2 and mean |err| <= 2e-3, and mean |err| <= 2% of
the output's RMS.

The bf16 throughput kernel (dh = 64, L > 128) is checked on inputs at std
0.5-1.0 (sharp_inputs): at the benchmark's own input scale (std 1/8) the
softmax is nearly uniform and a misaligned or missing position term stays
inside the tolerance, while on the sharp inputs it does not
(tests/test_parity_sensitivity.py).  The full-size configs are compared on
every output element.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_xl_relative_rel_amd as txl
from transformer_xl_relative_rel_amd import synth

from tests._common import check_close, late_rescale_fraction, sharp_inputs, spike_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV).to(dtype)


def run_gpu(d, dtype, **kw):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, r = (dev(d[x], td) for x in ("q", "k", "v", "r"))
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    out, lse = txl.relattn_fwd(q, k, v, r, u, vb, want_lse=True, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def config1_inputs():
    """B=1, H=2, dh=16, L=8, M=8, fp32; every random value 0.5*N(0,1); r_k is
    the sinusoid encoding of positions K-1..0 (d=32) times a random
    projection, split into heads."""
    B, H, L, M, dh = 1, 2, 8, 8, 16
    K, d = M + L, H * dh
    pe = oracle.pos_emb(K, d)                                   # [K, d]
    W_r = synth.normal((H * dh, d), synth.STREAM["w_r"], 0.5)
    r = (pe @ W_r.T).reshape(K, H, dh).transpose(1, 0, 2)       # [H, K, dh]
    return synth.relattn_inputs(B, H, L, M, dh, dtype="f32", std=0.5, bias_std=0.5, r_k=r)


def test_config1_fp32_full_parity():
    log("case: config1 fp32 B1 H2 dh16 L8 M8")
    d = config1_inputs()
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"])
    got, glse = run_gpu(d, "f32")
    check_close(got, want, "f32", "out")
    assert np.abs(glse - wlse).max() <= 1e-4


FP32_CASES = [
    # B, H, L, M, dh, splits
    (1, 1, 1, 0, 16, 0), (1, 2, 5, 0, 16, 0), (2, 3, 17, 3, 32, 0), (1, 2, 63, 1, 64, 0), (2, 4, 65, 64, 64, 0),
    (1, 8, 100, 37, 32, 0), (2, 4, 130, 200, 64, 3), (1, 1, 7, 150, 16, 5), (8, 1, 33, 31, 64, 1), (1, 3, 64, 0, 64, 2),
]


@pytest.mark.parametrize("B,H,L,M,dh,splits", FP32_CASES)
def test_fp32_parity_sweep(B, H, L, M, dh, splits):
    log(f"case: fp32 B{B} H{H} L{L} M{M} dh{dh} splits{splits}")
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="f32", std=0.5, bias_std=0.5, seed=1111 + L * 7 + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    got, glse = run_gpu(d, "f32", splits=splits)
    check_close(got, want, "f32", "out")
    assert np.abs(glse - wlse).max() <= 1e-4


BF16_CASES = [
    (1, 2, 1, 0, 64, 0), (2, 2, 19, 5, 32, 0), (1, 4, 128, 128, 64, 0), (2, 8, 200, 77, 64, 0),
    (1, 2, 96, 33, 128, 0), (2, 8, 256, 256, 64, 0), (1, 16, 128, 640, 64, 0), (1, 2, 70, 300, 64, 4),
    (4, 8, 256, 128, 64, 1),
    # B*H a multiple of 8 but H not: the XCD order by blocks of (b, h) pairs
    (4, 2, 160, 96, 64, 0), (2, 12, 150, 64, 64, 0),
]


@pytest.mark.parametrize("B,H,L,M,dh,splits", BF16_CASES)
def test_bf16_parity_sweep(B, H, L, M, dh, splits):
    log(f"case: bf16 B{B} H{H} L{L} M{M} dh{dh} splits{splits}")
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16", seed=2222 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    got, glse = run_gpu(d, "bf16", splits=splits)
    check_close(got, want, "bf16", "out")
    assert np.abs(glse - wlse).max() <= 2e-2


# The bf16 throughput kernel on inputs that separate a correct position term
# from a shifted or missing one.  splits = 1 keeps the kernel's own
# normalisation, 0 lets the plan split the keys (and run the combine).
SHARP_CASES = [
    # B, H, L, M, std, splits
    (1, 4, 160, 0, 1.0, 1),       # no memory; one pair group
    (2, 8, 160, 77, 0.5, 1),
    (2, 8, 300, 77, 0.7, 1),      # two pair groups, ragged last run
    (1, 8, 300, 512, 0.5, 0),     # automatic key split and combine
    (1, 8, 512, 256, 0.8, 1),
    (2, 8, 512, 512, 0.5, 1),     # the benchmark's L and M
    (1, 8, 512, 0, 1.0, 1),
    (4, 2, 160, 256, 0.6, 1),     # B*H a multiple of 8, H not: (b, h)-block XCD order
    (3, 5, 300, 77, 0.5, 1),      # neither: plain order
    (1, 8, 1000, 24, 0.5, 1),     # four pair groups
    (2, 8, 512, 512, 1.0, 3),     # forced key splits
]


@pytest.mark.parametrize("B,H,L,M,std,splits", SHARP_CASES)
def test_bf16_sharp_inputs_parity(B, H, L, M, std, splits):
    log(f"case: bf16 sharp B{B} H{H} L{L} M{M} std{std} splits{splits}")
    d = sharp_inputs(B, H, L, M, std, seed=500 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=16)
    got, glse = run_gpu(d, "bf16", splits=splits)
    check_close(got, want, "bf16", "out")
    assert np.abs(glse - wlse).max() <= 2e-2


@pytest.mark.parametrize("B,H,L,M,splits", [(2, 8, 512, 256, 1), (1, 8, 300, 512, 1), (2, 8, 160, 128, 1),
                                            (2, 8, 512, 512, 0)])
def test_bf16_late_dominant_key(B, H, L, M, splits):
    """A key after a query's first key tile beats everything it saw there by
    more than 8 log2 units (the online softmax must raise its maximum and
    rescale the accumulated output and denominator)."""
    log(f"case: bf16 late dominant key B{B} H{H} L{L} M{M} splits{splits}")
    d = spike_inputs(B, H, L, M, seed=600 + L + M)
    assert late_rescale_fraction(d, heads=2) >= 0.25
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=16)
    got, glse = run_gpu(d, "bf16", splits=splits)
    check_close(got, want, "bf16", "out")
    assert np.abs(glse - wlse).max() <= 2e-2


FULL = {
    "cfg2_B8_H16_dh64_L512_M256": (8, 16, 512, 256, 64),
    "cfg3_B8_H16_dh64_L512_M512": (8, 16, 512, 512, 64),
    "cfg4_B1_H16_dh64_L128_M1600": (1, 16, 128, 1600, 64),
}


@pytest.mark.parametrize("name", list(FULL))
@pytest.mark.parametrize("std", [None, 0.5])
def test_bf16_full_size_every_element(name, std):
    """Configs 2-4 at full size, every output and lse element against the
    oracle: once with the configs' own input scale (N(0,1)/8) and once with
    sharp inputs (std 0.5, u and vb 0.5)."""
    B, H, L, M, dh = FULL[name]
    log(f"case: {name} full tensor std {std}")
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16") if std is None else sharp_inputs(B, H, L, M, std, 700 + M)
    got, glse = run_gpu(d, "bf16")
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=16)
    check_close(got, want, "bf16", name)
    assert np.abs(glse - wlse).max() <= 2e-2


@pytest.mark.parametrize("dtype,dh", [("f32", 16), ("bf16", 32), ("bf16", 64)])
@pytest.mark.parametrize("L,M", [(8, 8), (5, 9), (3, 0)])
def test_mask_probe(dtype, dh, L, M):
    # q = u = vb = 0 and r = 0 make every visible score 0; v[j] = e_j shows which
    # keys each query sees: out[i][j] = 1/(M+i+1) if j <= i+M else exactly 0.
    log(f"case: mask probe {dtype} dh{dh} L{L} M{M}")
    K = M + L
    assert K <= dh
    z = np.zeros
    d = {"q": z((1, 1, L, dh)), "k": synth.normal((1, 1, K, dh), 2, 0.5), "v": np.eye(K, dh)[None, None],
         "r": z((1, K, dh)), "u": z((1, dh)), "vb": z((1, dh))}
    got, _ = run_gpu(d, dtype)
    vis = oracle.visible_mask(L, M)
    assert np.all((got[0, 0, :, :K] != 0) == vis)
    for i in range(L):
        np.testing.assert_allclose(got[0, 0, i, : i + M + 1], 1.0 / (i + M + 1), rtol=4e-3 if dtype == "bf16" else 1e-6)


DIST_CASES = [(dtype, dh, L, M, t) for dtype, dh in (("f32", 64), ("bf16", 64), ("bf16", 128))
              for L, M, t in ((16, 16, 0), (40, 70, 5), (64, 64, 33), (100, 20, 1))]
# the bf16 throughput kernel (L > 128): targets in the memory, in the segment, 0
DIST_CASES += [("bf16", 64, L, M, t) for L, M, t in ((256, 256, 100), (300, 512, 7), (512, 512, 0), (512, 512, 700),
                                                    (160, 0, 40))]


@pytest.mark.parametrize("dtype,dh,L,M,target", DIST_CASES)
def test_distance_probe(dtype, dh, L, M, target):
    # Only the position term is non-zero: vb = e_0 and r row c carries
    # -beta * |distance(c) - target| in column 0, distance(c) = K-1-c.  Each
    # query then attends (almost) only to the key at distance `target`,
    # j = i + M - target, or to key 0 when that key does not exist; v[j] = e_(j mod dh)
    # shows which key won.
    log(f"case: distance probe {dtype} dh{dh} L{L} M{M} target{target}")
    K = M + L
    beta = 64.0
    r = np.zeros((1, K, dh))
    r[0, :, 0] = -beta * np.abs(np.arange(K - 1, -1, -1) - target)
    vb = np.zeros((1, dh)); vb[0, 0] = 1.0
    v = np.zeros((1, 1, K, dh)); v[0, 0, np.arange(K), np.arange(K) % dh] = 1.0
    d = {"q": np.zeros((1, 1, L, dh)), "k": np.zeros((1, 1, K, dh)), "v": v, "r": r, "u": np.zeros((1, dh)), "vb": vb}
    got, _ = run_gpu(d, dtype)
    for i in range(L):
        j = max(i + M - target, 0)
        assert np.argmax(got[0, 0, i]) == j % dh, (i, j)
        assert got[0, 0, i, j % dh] > 0.99


def test_rows_sum_to_one_probe():
    log("case: row-sum probe bf16")
    d = synth.relattn_inputs(2, 4, 130, 70, 64, dtype="bf16")
    d["v"] = np.ones_like(d["v"])
    got, _ = run_gpu(d, "bf16")
    assert np.abs(got - 1.0).max() <= 4e-3


def test_strided_views_and_determinism():
    # q, k, v as views into one interleaved [B, T, 3, H, dh] buffer; out into a
    # [B, L, H, dh] buffer (the merged-heads layout).  Two runs are bitwise equal.
    log("case: strided views + determinism")
    B, H, L, M, dh = 2, 8, 96, 64, 64
    K = M + L
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16")
    buf = torch.zeros((B, K, 3, H, dh), dtype=torch.bfloat16, device=DEV)
    buf[:, :, 1] = dev(d["k"], torch.bfloat16).permute(0, 2, 1, 3)
    buf[:, :, 2] = dev(d["v"], torch.bfloat16).permute(0, 2, 1, 3)
    buf[:, M:, 0] = dev(d["q"], torch.bfloat16).permute(0, 2, 1, 3)
    q = buf[:, M:, 0].permute(0, 2, 1, 3)
    k = buf[:, :, 1].permute(0, 2, 1, 3)
    v = buf[:, :, 2].permute(0, 2, 1, 3)
    r = dev(d["r"], torch.bfloat16)
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    ob = torch.zeros((B, L, H, dh), dtype=torch.bfloat16, device=DEV)
    out = ob.permute(0, 2, 1, 3)
    txl.relattn_fwd(q, k, v, r, u, vb, out=out)
    torch.cuda.synchronize()
    first = ob.clone()
    txl.relattn_fwd(q, k, v, r, u, vb, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, ob)
    want, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    check_close(out.float().cpu().numpy(), want, "bf16", "strided")


def test_split_and_unsplit_agree():
    log("case: split vs unsplit")
    d = synth.relattn_inputs(1, 16, 128, 1600, 64, dtype="bf16")
    a, la = run_gpu(d, "bf16", splits=1)
    b, lb = run_gpu(d, "bf16", splits=0)
    # The two paths round p to bf16 against different running maxima, so they
    # agree to bf16 rounding, not bitwise; each is checked against the oracle
    # elsewhere.
    assert np.abs(a - b).max() <= 8e-3
    assert np.abs(la - lb).max() <= 1e-3
