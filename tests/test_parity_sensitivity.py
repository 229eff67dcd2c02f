"""The GPU parity tests of the bf16 throughput kernel can fail: on the inputs
they use, an output computed with the position term misaligned by one r row,
or without the position term at all, falls outside the bf16 tolerance.  The
planted mistakes are made in the oracle (on the CPU): the r rows are rolled
by one ([XL] "Transformer-XL", "Pitfall: Relative Shift Bugs Are
Shape-Correct": an off-by-one shift still runs) or zeroed, and the result is
rounded to bf16 like the kernel's output.

Also checks that the late-dominant-key inputs really require a rescale of the
online softmax (the deferred-rescale branch of the kernel), and that the
distance-probe recipe makes one key win at every query.
"""
import numpy as np
import pytest

import oracle
from transformer_xl_relative_rel_amd import synth

from tests._common import close_errors, late_rescale_fraction, sharp_inputs, spike_inputs

# (B, H, L, M, std, seed): shapes and scales of the GPU cases, fewer heads
CASES = [
    (1, 2, 160, 0, 1.0, 301),
    (1, 2, 160, 77, 0.5, 302),
    (1, 2, 300, 77, 0.7, 303),
    (1, 2, 512, 256, 0.8, 305),
    (1, 2, 512, 512, 0.5, 306),
]


def _rounded(out):
    return synth.round_bf16(out.astype(np.float32)).astype(np.float64)


@pytest.mark.parametrize("B,H,L,M,std,seed", CASES)
def test_position_term_bugs_fail_the_tolerance(B, H, L, M, std, seed):
    d = sharp_inputs(B, H, L, M, std, seed)
    want, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    assert not close_errors(_rounded(want), want, "bf16"), "the correct output must pass"
    for name, r in (("r off by one row", np.roll(d["r"], 1, axis=1)), ("r rows reversed", d["r"][:, ::-1]),
                    ("position term dropped", np.zeros_like(d["r"]))):
        bug, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], np.ascontiguousarray(r), d["u"], d["vb"], threads=8)
        assert close_errors(_rounded(bug), want, "bf16"), f"{name} passes the tolerance at {(B, H, L, M, std)}"


def test_default_scale_inputs_do_not_discriminate():
    """Why the sharp inputs exist: at the benchmark's own input scale an r row
    shift stays inside the tolerance (so those inputs cannot guard the
    position term on their own)."""
    d = synth.relattn_inputs(1, 2, 256, 256, 64, dtype="bf16")
    want, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    bug, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], np.roll(d["r"], 1, axis=1), d["u"], d["vb"], threads=8)
    assert not close_errors(_rounded(bug), want, "bf16")


@pytest.mark.parametrize("L,M", [(512, 256), (300, 512), (160, 128)])
def test_spike_inputs_force_a_late_rescale(L, M):
    d = spike_inputs(1, 2, L, M, seed=401 + L)
    frac = late_rescale_fraction(d)
    assert frac >= 0.25, frac
    # the non-dominant keys still carry weight: dropping them changes the output
    want, _ = oracle.relattn_fwd(d["q"], d["k"], d["v"], d["r"], d["u"], d["vb"], threads=8)
    ev = np.arange(0, L, 2)
    diff = np.abs(want[:, :, ev] - d["v"][:, :, M + ev]).mean()
    assert diff > 2e-2, diff
