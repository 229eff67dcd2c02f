"""Bit-exact parity of the HIP memory update (through the C ABI) with the
oracle's Tail_M, over several consecutive segments."""
import numpy as np
import pytest
import torch

import oracle
import transformer_xl_relative_rel_amd as txl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    """Raw bytes of a device tensor as a numpy uint8 array."""
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _segments(B, L, d, n, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn((B, L, d), generator=g).to(dtype) for _ in range(n)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L,M,ext", [(8, 8, 0), (3, 8, 0), (12, 8, 0), (3, 0, 0), (12, 0, 0), (5, 17, 0), (6, 5, 2)])
def test_mem_update_matches_oracle_over_segments(dtype, L, M, ext):
    print(f"case: mem_update {dtype} L{L} M{M} ext{ext}", flush=True)
    B, d = 2, 32
    segs = _segments(B, L, d, 4, dtype, seed=L * 13 + M)
    mem_g, mem_o = None, None
    npd = np.float32 if dtype == torch.float32 else np.uint16
    for s in segs:
        new_g = txl.mem_update(mem_g, s.to(DEV), M, ext_len=ext)
        torch.cuda.synchronize()
        h_np = s.view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 else s.numpy()
        mem_o = oracle.mem_update(mem_o, h_np.astype(npd, copy=False), M, ext_len=ext)
        assert tuple(new_g.shape) == mem_o.shape
        np.testing.assert_array_equal(_bits(new_g), mem_o.view(np.uint8).reshape(_bits(new_g).shape))
        mem_g = new_g


def test_batched_update_matches_single():
    print("case: mem_update batched 17 buffers", flush=True)
    B, L, M, d, n = 4, 64, 48, 256, 17
    hs = [t.to(DEV) for t in _segments(B, L, d, n, torch.bfloat16, seed=3)]
    m0 = [t.to(DEV) for t in _segments(B, M, d, n, torch.bfloat16, seed=4)]
    outs = txl.mem_update_batched(m0, hs, M)
    singles = [txl.mem_update(m, h, M) for m, h in zip(m0, hs)]
    torch.cuda.synchronize()
    for a, b in zip(outs, singles):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_full_size_update_is_exact_tail():
    # One 16-layer-stack memory: B=4, M=512, d=1024, bf16; tail of [mem; h].
    print("case: mem_update full size", flush=True)
    B, L, M, d = 4, 512, 512, 1024
    mem = torch.randn((B, M, d), device=DEV).to(torch.bfloat16)
    h = torch.randn((B, L, d), device=DEV).to(torch.bfloat16)
    new = txl.mem_update(mem, h, M)
    torch.cuda.synchronize()
    want = torch.cat([mem, h], 1)[:, -M:]
    assert torch.equal(new.view(torch.int16), want.view(torch.int16))
