"""Decoder layer (txl_layer_fwd) and a small layer stack on the GPU against the
CPU oracle's post-LN layer (oracle.layer_fwd, [SRC] RelPartialLearnableDecoderLayer
with pre_lnorm = False).

Inputs, weights and memories are rounded to bf16 first and the oracle runs in
fp64 on those exact values.  Tolerance (the layer outputs are LayerNorm
outputs of unit scale, |y| < 5 here): the GPU rounds to bf16 six
intermediates on the way (position table, r_k / q / k / v, P, the merged
heads, LN1 output, the ReLU output), each to within 2^-9 relative, and the
result once more (2^-9 |y| <= 0.0098).  Summed worst case 6 * 2^-9 = 1.2 % of
the normalised magnitude, i.e. <= 0.06 absolute for |y| < 5; the mean error of
independent roundings is about sqrt(6) * 2^-9 / sqrt(3) of the RMS (~0.003).
Bounds: max |err| <= 6e-2, mean |err| <= 5e-3.
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
MAX_ERR, MEAN_ERR = 6e-2, 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rnd(shape, stream, std):
    return synth.round_bf16(synth.normal(shape, stream, std))


def make_layer(d, H, dh, di, seed):
    """Random layer weights (bf16-exact matrices, fp32 vectors)."""
    HD = H * dh
    w = {
        "W_qkv": rnd((3 * HD, d), seed + 1, 1.0 / np.sqrt(d)),
        "W_r": rnd((HD, d), seed + 2, 1.0 / np.sqrt(d)),
        "W_o": rnd((d, HD), seed + 3, 1.0 / np.sqrt(HD)),
        "ln1_g": 1.0 + synth.normal((d,), seed + 4, 0.1),
        "ln1_b": synth.normal((d,), seed + 5, 0.1),
        "W1": rnd((di, d), seed + 6, 1.0 / np.sqrt(d)),
        "b1": synth.normal((di,), seed + 7, 0.1),
        "W2": rnd((d, di), seed + 8, 1.0 / np.sqrt(di)),
        "b2": synth.normal((d,), seed + 9, 0.1),
        "ln2_g": 1.0 + synth.normal((d,), seed + 10, 0.1),
        "ln2_b": synth.normal((d,), seed + 11, 0.1),
    }
    return {k: np.asarray(v, dtype=np.float32).astype(np.float64) for k, v in w.items()}


def to_dev(w):
    out = {}
    for k, v in w.items():
        t = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(DEV)
        out[k] = t.to(torch.bfloat16) if v.ndim == 2 else t
    return out


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(torch.bfloat16)


def check(got, want, what):
    err = np.abs(got - want)
    log(f"  {what}: max err {err.max():.3e} mean {err.mean():.3e} (|want| max {np.abs(want).max():.2f})")
    assert err.max() <= MAX_ERR, f"{what}: max err {err.max():.3e}"
    assert err.mean() <= MEAN_ERR, f"{what}: mean err {err.mean():.3e}"


@pytest.mark.parametrize("B,L,M_cur,d,H,dh,di", [
    (2, 16, 0, 128, 2, 64, 256),      # first segment: no memory
    (2, 16, 16, 128, 2, 64, 256),
    (1, 40, 24, 256, 4, 64, 512),     # ragged L, memory shorter than L
    (2, 8, 32, 128, 4, 32, 128),      # dh = 32 (generic attention kernel)
    (1, 16, 8, 256, 2, 128, 256),     # dh = 128
])
def test_layer_matches_oracle(B, L, M_cur, d, H, dh, di):
    log(f"case: layer B{B} L{L} M{M_cur} d{d} H{H} dh{dh} di{di}")
    w = make_layer(d, H, dh, di, 100 + d + dh)
    h = rnd((B, L, d), 7, 1.0).astype(np.float64)
    mem = rnd((B, M_cur, d), 8, 1.0).astype(np.float64) if M_cur else None
    u = synth.normal((H, dh), 9, 0.5)
    vb = synth.normal((H, dh), 10, 0.5)
    want = oracle.layer_fwd(h, mem, w, u, vb, H, dh)
    tu = torch.from_numpy(np.asarray(u, np.float32)).to(DEV)
    tv = torch.from_numpy(np.asarray(vb, np.float32)).to(DEV)
    got = txl.layer_fwd(bf(h), bf(mem) if M_cur else None, to_dev(w), tu, tv, H, dh)
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), want, "layer out")


def test_layer_is_deterministic():
    log("case: layer determinism")
    B, L, M_cur, d, H, dh, di = 2, 32, 32, 128, 2, 64, 256
    w = to_dev(make_layer(d, H, dh, di, 5))
    h, mem = bf(rnd((B, L, d), 1, 1.0)), bf(rnd((B, M_cur, d), 2, 1.0))
    u = torch.full((H, dh), 0.1, device=DEV)
    a = txl.layer_fwd(h, mem, w, u, u, H, dh)
    b = txl.layer_fwd(h, mem, w, u, u, H, dh)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_stack_segments_against_oracle():
    """Two layers over three segments of L=16 with mem_len=16 ([SRC]
    MemTransformerLM._forward / _update_mems): every layer output is checked
    against the oracle layer on the same (GPU) inputs and memories, and every
    memory buffer is checked bit-exactly against Tail_M of [old memory; layer
    input]."""
    log("case: 2-layer stack, 3 segments")
    B, L, d, H, dh, di, mem_len, n_layer = 2, 16, 128, 2, 64, 256, 16, 2
    layers = [make_layer(d, H, dh, di, 1000 * (n + 1)) for n in range(n_layer)]
    dlayers = [to_dev(w) for w in layers]
    u = synth.normal((H, dh), 21, 0.5)
    vb = synth.normal((H, dh), 22, 0.5)
    tu = torch.from_numpy(np.asarray(u, np.float32)).to(DEV)
    tv = torch.from_numpy(np.asarray(vb, np.float32)).to(DEV)
    mems = [None] * (n_layer + 1)
    for seg in range(3):
        x = bf(rnd((B, L, d), 300 + seg, 1.0))
        hids = [x]
        for n in range(n_layer):
            hids.append(txl.layer_fwd(hids[n], mems[n], dlayers[n], tu, tv, H, dh))
        torch.cuda.synchronize()
        for n in range(n_layer):
            m = None if mems[n] is None else mems[n].float().cpu().numpy().astype(np.float64)
            want = oracle.layer_fwd(hids[n].float().cpu().numpy().astype(np.float64), m, layers[n], u, vb, H, dh)
            check(hids[n + 1].float().cpu().numpy(), want, f"segment {seg} layer {n}")
        new = txl.mem_update_batched(mems if mems[0] is not None else None, hids, mem_len)
        torch.cuda.synchronize()
        for n in range(n_layer + 1):
            old = None if mems[n] is None else mems[n].view(torch.int16).cpu().numpy()
            want = oracle.mem_update(old, hids[n].view(torch.int16).cpu().numpy(), mem_len)
            assert np.array_equal(new[n].view(torch.int16).cpu().numpy(), want)
        mems = new


@pytest.mark.parametrize("clamp_len,same_length,mem_valid", [(5, 0, None), (0, 20, None), (0, 0, [0, 9]),
                                                             (7, 24, [16, 3])])
def test_layer_options_match_oracle(clamp_len, same_length, mem_valid):
    """clamp_len, same_length and per-row memory validity against the oracle layer."""
    B, L, M_cur, d, H, dh, di = 2, 24, 16, 128, 2, 64, 256
    log(f"case: layer options clamp{clamp_len} same_length{same_length} mem_valid{mem_valid}")
    w = make_layer(d, H, dh, di, 31)
    h = rnd((B, L, d), 32, 1.0).astype(np.float64)
    mem = rnd((B, M_cur, d), 33, 1.0).astype(np.float64)
    u = synth.normal((H, dh), 34, 0.5)
    vb = synth.normal((H, dh), 35, 0.5)
    want = oracle.layer_fwd(h, mem, w, u, vb, H, dh, clamp_len=clamp_len, same_length=same_length,
                            mem_valid=mem_valid)
    tu = torch.from_numpy(np.asarray(u, np.float32)).to(DEV)
    tv = torch.from_numpy(np.asarray(vb, np.float32)).to(DEV)
    mv = None if mem_valid is None else torch.tensor(mem_valid, dtype=torch.int32, device=DEV)
    got = txl.layer_fwd(bf(h), bf(mem), to_dev(w), tu, tv, H, dh, clamp_len=clamp_len, same_length=same_length,
                        mem_valid=mv)
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), want, "layer out")


def test_stack_with_per_row_resets():
    """Two layers over four segments of three streams; rows 0 and 2 start new
    documents at segments 2 and 1.  The device keeps full memory buffers and a
    per-row count of valid memory rows; every layer output of every row must
    equal the oracle layer run on that row alone with only its valid memory
    ([XL] "Batched Streams": memory belongs to the row's own stream)."""
    log("case: 2-layer stack, 4 segments, per-row resets")
    B, L, d, H, dh, di, mem_len, n_layer = 3, 16, 128, 2, 64, 256, 24, 2
    resets = {1: [2], 2: [0]}
    layers = [make_layer(d, H, dh, di, 500 * (n + 1)) for n in range(n_layer)]
    dlayers = [to_dev(w) for w in layers]
    u = synth.normal((H, dh), 41, 0.5)
    vb = synth.normal((H, dh), 42, 0.5)
    tu = torch.from_numpy(np.asarray(u, np.float32)).to(DEV)
    tv = torch.from_numpy(np.asarray(vb, np.float32)).to(DEV)
    mems = [None] * (n_layer + 1)
    valid = [0] * B
    for seg in range(4):
        for b in resets.get(seg, []):
            valid[b] = 0
        M_cur = 0 if mems[0] is None else mems[0].shape[1]
        mv = torch.tensor([min(v, M_cur) for v in valid], dtype=torch.int32, device=DEV)
        x = bf(rnd((B, L, d), 600 + seg, 1.0))
        hids = [x]
        for n in range(n_layer):
            hids.append(txl.layer_fwd(hids[n], mems[n], dlayers[n], tu, tv, H, dh,
                                      mem_valid=mv if M_cur else None))
        torch.cuda.synchronize()
        for n in range(n_layer):
            hin = hids[n].float().cpu().numpy().astype(np.float64)
            for b in range(B):
                m = min(valid[b], M_cur)
                mem_b = None if m == 0 else mems[n][b:b + 1, M_cur - m:].float().cpu().numpy().astype(np.float64)
                want = oracle.layer_fwd(hin[b:b + 1], mem_b, layers[n], u, vb, H, dh)
                check(hids[n + 1][b:b + 1].float().cpu().numpy(), want, f"segment {seg} layer {n} row {b}")
        mems = txl.mem_update_batched(mems if mems[0] is not None else None, hids, mem_len)
        torch.cuda.synchronize()
        valid = [min(mems[0].shape[1], v + L) for v in valid]
