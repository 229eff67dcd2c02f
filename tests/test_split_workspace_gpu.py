"""Key-split calls with the workspace, out and lse pre-filled with NaN bytes.

A split call writes every row's partial (O, m, l) to the workspace, including
rows that see no key in the split (o = 0, l = 0, m = -inf), and the combine
reads every split of every row ([SRC] RelPartialLearnableMultiHeadAttn.forward,
softmax over the whole key axis, evaluated here as an exact merge of per-split
partial softmaxes).  With the buffers filled with 0xFF bytes (fp32 NaN, bf16
NaN) a read of anything not written first shows up as a non-finite or wrong
output.  Each case runs the path its shape selects (throughput kernel, streaming
kernel, masked instances, the fp32 generic kernel) against the oracle with the
tolerances of the other parity modules.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_xl_relative_rel_amd as txl
from transformer_xl_relative_rel_amd import synth

from tests._common import check_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


CASES = [
    # dtype, B, H, L, M, dh, splits, window, mem_valid
    ("bf16", 2, 4, 300, 200, 64, 3, 0, None),          # throughput kernel, three key ranges
    ("bf16", 1, 16, 128, 1600, 64, 0, 0, None),        # streaming kernel, automatic split plan
    ("bf16", 1, 16, 40, 700, 64, 5, 0, None),          # streaming kernel, ragged run
    ("bf16", 2, 2, 200, 300, 64, 4, 120, [40, 300]),   # masked instances: window and hidden memory
    ("bf16", 1, 2, 70, 300, 32, 3, 0, [10]),           # generic bf16 kernel (dh 32)
    ("f32", 2, 3, 50, 30, 16, 2, 0, None),             # fp32 generic kernel
    ("f32", 1, 2, 65, 200, 64, 4, 64, [100]),
]


@pytest.mark.parametrize("dtype,B,H,L,M,dh,splits,window,mem_valid", CASES)
def test_split_call_reads_only_what_it_wrote(dtype, B, H, L, M, dh, splits, window, mem_valid):
    log(f"case: {dtype} B{B} H{H} L{L} M{M} dh{dh} splits{splits} window{window} mem_valid{mem_valid}")
    d = synth.relattn_inputs(B, H, L, M, dh, dtype=dtype, std=0.5, bias_std=0.5, seed=4242 + L + M)
    want, wlse = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8,
                                    same_length=window, mem_valid=mem_valid)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, r = (dev(d[x], td) for x in ("q", "k", "v", "r"))
    u, vb = dev(d["u"], torch.float32), dev(d["vb"], torch.float32)
    mv = None if mem_valid is None else torch.tensor(mem_valid, dtype=torch.int32, device=DEV)
    nbytes = txl.relattn_workspace_size(q, k, splits=splits)
    ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.full(q.shape, float("nan"), dtype=td, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    txl.relattn_fwd(q, k, v, r, u, vb, out=out, lse=lse, splits=splits, workspace=ws, window=window, mem_valid=mv)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    glse = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(glse)), "unwritten or NaN-contaminated output"
    check_close(got, want, dtype, "out")
    assert np.abs(glse - wlse).max() <= (1e-4 if dtype == "f32" else 2e-2)
