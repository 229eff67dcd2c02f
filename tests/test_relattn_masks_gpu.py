"""Mask variants of the HIP relative attention against the CPU oracle: the
same_length window ([SRC] MemTransformerLM._forward, same_length=True) and
per-row memory validity after a document boundary ([XL] "Batched Streams").

The kernel takes the window as `window` (query i sees keys j >= i + M + 1 -
window) and the oracle builds the page's literal triu + tril mask with
mem_len = window; the two meet only in the results.  Tolerances as in
test_relattn_gpu.py (fp32 1e-4; bf16 2e-2 max, 2e-3 mean, 2% of the RMS).
"""
import math
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


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def run_gpu(d, dtype, window=0, mem_valid=None, splits=0):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, r = (dev(d[x], td) for x in ("q", "k", "v", "r"))
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    mv = None if mem_valid is None else torch.tensor(mem_valid, dtype=torch.int32, device=DEV)
    out, lse = txl.relattn_fwd(q, k, v, r, u, vb, want_lse=True, window=window, mem_valid=mv, splits=splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    # dtype, B, H, L, M, dh, window, mem_valid, splits
    ("bf16", 2, 4, 300, 200, 64, 0, [0, 117], 0),
    ("bf16", 2, 4, 300, 200, 64, 64, None, 0),
    ("bf16", 2, 4, 300, 200, 64, 250, [50, 200], 0),
    ("bf16", 1, 8, 512, 512, 64, 512, [100], 0),     # same_length with a full memory
    ("bf16", 2, 4, 256, 64, 64, 1, [64, 0], 0),      # window 1: each query sees only itself
    ("bf16", 1, 2, 70, 300, 64, 100, [30], 4),       # key-range splits
    ("bf16", 2, 2, 40, 24, 32, 16, [0, 24], 0),
    ("bf16", 1, 2, 33, 40, 128, 20, [7], 0),
    ("f32", 2, 3, 50, 30, 16, 9, [0, 11], 0),
    ("f32", 1, 2, 65, 64, 64, 64, [64], 2),
    ("f32", 2, 1, 17, 0, 32, 5, [0, 0], 0),          # no memory at all
]


@pytest.mark.parametrize("dtype,B,H,L,M,dh,window,mem_valid,splits", CASES)
def test_mask_variant_parity(dtype, B, H, L, M, dh, window, mem_valid, splits):
    log(f"case: {dtype} B{B} H{H} L{L} M{M} dh{dh} window{window} mem_valid{mem_valid} splits{splits}")
    if dtype == "f32":
        d = synth.relattn_inputs(B, H, L, M, dh, dtype="f32", std=0.5, bias_std=0.5, seed=77 + L + M)
    else:
        d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16", seed=88 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8,
                                    same_length=window, mem_valid=mem_valid)
    got, glse = run_gpu(d, dtype, window=window, mem_valid=mem_valid, splits=splits)
    check_close(got, want, dtype, "out")
    assert np.abs(glse - wlse).max() <= (1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("dh", [32, 64])
def test_first_visible_tile_sets_the_max(dh):
    # Every score carries a common offset of about -144 log2 units (u[0] = -800
    # against k[:, 0] = 1), and the window hides the first key tiles from the
    # later queries of each block.  A query whose running max stayed at its
    # initial value through those hidden tiles would underflow exp2 on its
    # first visible tile and divide 0 by 0; the exact max of the first visible
    # tile keeps every row finite and equal to the oracle.
    B, H, L, M, window = 2, 2, 300, 100, 40
    log(f"case: far negative scores, bf16 dh{dh} window{window}")
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16", seed=99)
    d["k"][..., 0] = 1.0
    d["u"][:, 0] = -800.0
    want, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8, same_length=window,
                                 mem_valid=[M, 3])
    got, _ = run_gpu(d, "bf16", window=window, mem_valid=[M, 3])
    check_close(got, want, "bf16", "out")


@pytest.mark.parametrize("std", [None, 0.5])
def test_headline_shape_with_masks_every_element(std):
    # B=8, H=16, dh=64, L=512, M=512 with same_length (window 512) and a
    # different valid-memory count per batch row; every element against the
    # oracle, at the config's input scale and with sharp inputs.
    B, H, L, M, dh, window = 8, 16, 512, 512, 64, 512
    mv = [0, 1, 63, 64, 200, 511, 512, 300]
    log(f"case: headline shape with window 512 and per-row memory validity, std {std}")
    d = synth.relattn_inputs(B, H, L, M, dh, dtype="bf16") if std is None else sharp_inputs(B, H, L, M, std, 901)
    got, glse = run_gpu(d, "bf16", window=window, mem_valid=mv)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=16,
                                    same_length=window, mem_valid=mv)
    check_close(got, want, "bf16", "full tensor")
    assert np.abs(glse - wlse).max() <= 2e-2


SHARP_MASK_CASES = [
    # B, H, L, M, std, window, mem_valid, splits
    (2, 8, 300, 200, 0.7, 0, [0, 117], 1),
    (2, 8, 300, 200, 0.5, 64, None, 1),
    (2, 8, 512, 512, 0.5, 300, [40, 512], 1),
    (1, 8, 512, 256, 1.0, 1, None, 1),
    (2, 8, 160, 77, 0.6, 100, [77, 5], 0),
]


@pytest.mark.parametrize("B,H,L,M,std,window,mem_valid,splits", SHARP_MASK_CASES)
def test_mask_variant_sharp_inputs(B, H, L, M, std, window, mem_valid, splits):
    log(f"case: masked bf16 sharp B{B} H{H} L{L} M{M} std{std} window{window} mem_valid{mem_valid} splits{splits}")
    d = sharp_inputs(B, H, L, M, std, seed=950 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=16,
                                    same_length=window, mem_valid=mem_valid)
    got, glse = run_gpu(d, "bf16", window=window, mem_valid=mem_valid, splits=splits)
    check_close(got, want, "bf16", "out")
    assert np.abs(glse - wlse).max() <= 2e-2


@pytest.mark.parametrize("L,M,window,target", [(300, 200, 250, 100), (512, 512, 512, 300), (256, 64, 100, 0),
                                               (512, 256, 200, 199)])
def test_distance_probe_with_window(L, M, window, target):
    """[XL] "Relative Shift Golden Test" through the masked throughput kernel:
    only the position term is non-zero and r row c scores -64 |distance(c) -
    target| (distance(c) = K-1-c), so every query attends to the key at
    distance `target`, j = i + M - target, which the window keeps visible
    (target < window, target <= M); v[j] = e_(j mod 64) shows which key won."""
    log(f"case: distance probe with window L{L} M{M} window{window} target{target}")
    K, dh = M + L, 64
    r = np.zeros((1, K, dh))
    r[0, :, 0] = -64.0 * np.abs(np.arange(K - 1, -1, -1) - target)
    vb = np.zeros((1, dh)); vb[0, 0] = 1.0
    v = np.zeros((1, 1, K, dh)); v[0, 0, np.arange(K), np.arange(K) % dh] = 1.0
    d = {"q": np.zeros((1, 1, L, dh)), "k": np.zeros((1, 1, K, dh)), "v": v, "r": r, "u": np.zeros((1, dh)), "vb": vb}
    got, _ = run_gpu(d, "bf16", window=window, splits=1)
    for i in range(L):
        j = i + M - target
        assert np.argmax(got[0, 0, i]) == j % dh, (i, j)
        assert got[0, 0, i, j % dh] > 0.99


def test_invalid_window_is_rejected():
    d = synth.relattn_inputs(1, 1, 4, 2, 64, dtype="bf16")
    with pytest.raises(txl.TxlError, match="window"):
        run_gpu(d, "bf16", window=-1)
