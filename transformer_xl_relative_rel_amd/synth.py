"""Seeded synthetic inputs.

This module holds no part of the attention arithmetic: it only draws
reproducible random numbers and rounds them to the storage type.  Both the
device path and the CPU reference are fed from it.

Generator (defined here, not taken from any library):
  * counter-based splitmix64: the n-th 64-bit word of stream s under seed S is
    mix64(S + (s * 2**40 + n + 1) * 0x9E3779B97F4A7C15) with the usual
    splitmix64 finaliser (xor-shift 30 / 27 / 31, multipliers
    0xBF58476D1CE4E5B9 and 0x94D049BB133111EB);
  * uniforms from the top 53 bits: (w >> 11) * 2**-53, shifted to (0, 1] for
    the logarithm;
  * Box-Muller: words 2t and 2t+1 give u1, u2 and the pair
    sqrt(-2 ln u1) * (cos 2 pi u2, sin 2 pi u2);
  * bf16 rounding: round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SEED = 1111


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def words(n: int, stream: int, seed: int = SEED) -> np.ndarray:
    """n splitmix64 words of a stream (uint64)."""
    with np.errstate(over="ignore"):
        ctr = np.arange(1, n + 1, dtype=np.uint64) + np.uint64(stream << 40)
        return _mix64(np.uint64(seed) + ctr * GOLDEN)


def uniform(n: int, stream: int, seed: int = SEED) -> np.ndarray:
    """n doubles in [0, 1)."""
    return (words(n, stream, seed) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(shape, stream: int, std: float = 1.0, seed: int = SEED) -> np.ndarray:
    """float64 array of N(0, std^2) samples via Box-Muller."""
    n = int(np.prod(shape))
    pairs = (n + 1) // 2
    w = words(2 * pairs, stream, seed)
    u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)   # (0, 1]
    u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)           # [0, 1)
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * pairs, dtype=np.float64)
    z[0::2] = rad * np.cos(2.0 * np.pi * u2)
    z[1::2] = rad * np.sin(2.0 * np.pi * u2)
    return (z[:n] * std).reshape(shape)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32 holding bf16 values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(f.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values that are already bf16-representable."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# Fixed stream numbers, one per tensor role, so every consumer draws the same values.
STREAM = {"q": 1, "k": 2, "v": 3, "r": 4, "u": 5, "vb": 6, "h": 7, "mem": 8, "w_r": 9, "emb": 10, "dout": 11}


def relattn_inputs(B: int, H: int, L: int, M: int, dh: int, dtype: str = "bf16",
                   std: float | None = None, bias_std: float = 0.02, seed: int = SEED,
                   r_k: np.ndarray | None = None) -> dict:
    """Inputs of one relative-attention call as float32 arrays.

    q [B, H, L, dh]; k, v [B, H, M+L, dh]; r [H, M+L, dh]; u, vb [H, dh].
    Activations are N(0, std^2) (std defaults to 1/sqrt(dh)); u and vb are
    N(0, bias_std^2) and stay float32.  With dtype 'bf16' the activations are
    rounded to bf16 values.  ``r_k`` replaces the drawn r when given.
    """
    K = M + L
    sd = (1.0 / np.sqrt(dh)) if std is None else std
    out = {
        "q": normal((B, H, L, dh), STREAM["q"], sd, seed),
        "k": normal((B, H, K, dh), STREAM["k"], sd, seed),
        "v": normal((B, H, K, dh), STREAM["v"], sd, seed),
        "r": normal((H, K, dh), STREAM["r"], sd, seed) if r_k is None else np.asarray(r_k, np.float64),
        "u": normal((H, dh), STREAM["u"], bias_std, seed),
        "vb": normal((H, dh), STREAM["vb"], bias_std, seed),
    }
    for key in ("q", "k", "v", "r"):
        a = out[key].astype(np.float32)
        out[key] = round_bf16(a) if dtype == "bf16" else a
    for key in ("u", "vb"):
        out[key] = out[key].astype(np.float32)
    return out
