"""The full-size layer stack (16 post-LN layers, d = 1024, H = 16, d_inner =
4096, B = 4, eight segments of L = 512 with mem_len = 512; weights N(0, 0.02),
LayerNorm gamma = 1, beta = 0, biases 0, embeddings N(0, 1)), which no CPU
reference can run at this size.  It is pinned by invariants that hold at any
size ([SRC] MemTransformerLM._forward / _update_mems; [XL] "Segment-Level
Recurrence"):
  * every memory buffer after a segment is the tail of [old memory; the
    layer's input], bit for bit (with L = mem_len: exactly the input);
  * every layer output is a LayerNorm output with gamma = 1, beta = 0: each
    row has mean 0 and (biased) variance 1, up to the bf16 rounding of the
    stored output (2^-9 relative per element: |mean| <= 5e-3,
    |var - 1| <= 2e-2) and eps / var (< 1e-4 here);
  * nothing is NaN or Inf;
  * the memory is used: the second segment's output changes when its memory
    is replaced by zeros of the same shape.
The layer arithmetic itself is compared with the oracle at reduced shapes in
test_layer_gpu.py.
"""
import sys

import pytest
import torch

import transformer_xl_relative_rel_amd as txl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_LAYER, D, H, DH, DI, B, L, MEM, SEGS = 16, 1024, 16, 64, 4096, 4, 512, 512, 8


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_stack(gen):
    def w(*shape):
        return (torch.randn(*shape, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)

    layers = []
    for _ in range(N_LAYER):
        layers.append({"W_qkv": w(3 * H * DH, D), "W_r": w(H * DH, D), "W_o": w(D, H * DH),
                       "ln1_g": torch.ones(D, device=DEV), "ln1_b": torch.zeros(D, device=DEV),
                       "W1": w(DI, D), "b1": torch.zeros(DI, device=DEV), "W2": w(D, DI),
                       "b2": torch.zeros(D, device=DEV), "ln2_g": torch.ones(D, device=DEV),
                       "ln2_b": torch.zeros(D, device=DEV)})
    u = torch.randn(H, DH, generator=gen, device=DEV) * 0.02
    vb = torch.randn(H, DH, generator=gen, device=DEV) * 0.02
    return layers, u, vb


def test_stack_config5_invariants():
    log("case: 16-layer stack, B4 d1024 H16 d_inner 4096, 8 segments of L512, mem_len 512")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1111)
    layers, u, vb = make_stack(gen)
    mems = None
    seg2_in = None
    for seg in range(SEGS):
        x = torch.randn(B, L, D, generator=gen, device=DEV).to(torch.bfloat16)
        old = mems
        hids, mems = txl.stack_segment(x, mems, layers, u, vb, H, DH, MEM)
        torch.cuda.synchronize()
        worst_mean = worst_var = 0.0
        for n in range(1, N_LAYER + 1):
            y = hids[n].float()
            assert torch.isfinite(y).all(), f"segment {seg} layer {n - 1}: non-finite output"
            worst_mean = max(worst_mean, y.mean(dim=-1).abs().max().item())
            worst_var = max(worst_var, (y.var(dim=-1, unbiased=False) - 1.0).abs().max().item())
        log(f"  segment {seg}: max |row mean| {worst_mean:.2e}, max |row var - 1| {worst_var:.2e}")
        assert worst_mean <= 5e-3 and worst_var <= 2e-2
        for n in range(N_LAYER + 1):
            assert mems[n].shape == (B, MEM, D)
            assert torch.equal(mems[n].view(torch.int16), hids[n].view(torch.int16)), f"memory {n} != input of layer {n}"
        if seg == 1:
            seg2_in, seg2_out, seg2_mems = x, hids[-1].clone(), [m.clone() for m in old]
    # the second segment again, with zero memories of the same shape
    zero = [torch.zeros_like(m) for m in seg2_mems]
    hz, _ = txl.stack_segment(seg2_in, zero, layers, u, vb, H, DH, MEM)
    torch.cuda.synchronize()
    diff = (hz[-1].float() - seg2_out.float()).abs().max().item()
    log(f"  segment 1 output with zeroed memory differs by {diff:.3e}")
    assert diff > 1e-2
