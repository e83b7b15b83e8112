"""Number formats of the 4-bit path, written out from their definitions.

Test infrastructure (see the package docstring): only tests, the smoke check and
the benchmark's CPU baseline use this module.

* E2M1 (FP4): the eight magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3
  of the nibble.  "Getting GLM-5.2 NVFP4 Post-Training off the ground", section
  "Why can't we just transpose the one copy?" (4-bit E2M1 values with a
  per-16-element FP8 E4M3 scale and one FP32 global scale); the largest
  magnitude 6 is the E2M1_MAX of "The 4-bitter Lesson", section "Four-Over-Six
  for RL Weights and Activations".
* E4M3 (the OCP "FN" variant): bias 7, three mantissa bits, largest finite 448,
  smallest subnormal 2^-9, no infinities, 0x7F is NaN.
* bf16: the top half of an IEEE float32, rounded to nearest even.
* NF4: the 16-level NormalFloat codebook of QLoRA, named with blocksize 64 in
  "nf4moe - QLoRA for a 743B Fused-MoE", section "The fix: dequant-on-forward
  for routed experts".  The pages never print the 16 values: parity unpinned
  for them.  They are built here from the NormalFloat construction (quantiles
  of N(0,1), 8 positive and 7 negative levels plus an exact zero, normalised
  to [-1, 1]).  The one free constant is the probability of the outermost
  quantile, taken as the mean of 1 - 1/(2*15) and 1 - 1/(2*16).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# E2M1 magnitudes, code 0..7.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
E2M1_MAX = F32(6.0)
E4M3_MAX = F32(448.0)


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------
def bf16_rne_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Finite inputs only.  The 16 discarded bits are rounded into the kept half:
    add 0x7FFF plus the lowest kept bit, then truncate.
    """
    u = f32(x).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """float32 (or float64, first rounded to float32) -> nearest bf16 value, as float32."""
    return bf16_bits_to_f32(bf16_rne_bits(f32(x)))


# ----------------------------------------------------------------------------
# E4M3 (FN) block scales
# ----------------------------------------------------------------------------
def e4m3_rne_satfinite(t) -> np.ndarray:
    """Non-negative float32 -> E4M3FN bit pattern (uint8).

    Round to nearest, ties to even, on the E4M3 grid; anything that would round
    above 448 saturates to 448.  Below 2^-6 the grid is the subnormal step 2^-9.
    """
    t64 = f32(t).astype(np.float64)
    if np.any(t64 < 0) or not np.all(np.isfinite(t64)):
        raise ValueError("e4m3_rne_satfinite expects finite non-negative input")
    # exponent of the binade [2^e, 2^(e+1)); subnormal range uses e = -6
    _, ex = np.frexp(t64)            # t = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    step = np.ldexp(1.0, (e - 3).astype(np.int64))   # 3 mantissa bits
    q = np.rint(t64 / step) * step                     # rint: ties to even
    q = np.minimum(q, 448.0)
    # encode q (exact on the grid now)
    out = np.zeros(q.shape, dtype=np.uint8)
    nz = q > 0
    qn = q[nz]
    _, ex2 = np.frexp(qn)
    e2 = ex2.astype(np.int64) - 1
    sub = e2 < -6
    mant_sub = np.rint(qn / 2.0 ** -9).astype(np.int64)          # 1..7
    frac = np.rint((qn / np.ldexp(1.0, e2) - 1.0) * 8).astype(np.int64)  # 0..7
    code = np.where(sub, mant_sub, ((e2 + 7) << 3) | frac)
    out[nz] = code.astype(np.uint8)
    return out


def e4m3_decode(bits) -> np.ndarray:
    """E4M3FN bit pattern -> float32 (sign honoured; 0x7F / 0xFF give NaN)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return (s * val).astype(np.float32)


# ----------------------------------------------------------------------------
# E2M1 element codes
# ----------------------------------------------------------------------------
def e2m1_mag_code(v) -> np.ndarray:
    """Non-negative float32 -> E2M1 magnitude code 0..7, nearest, ties to even code.

    The midpoints between neighbouring grid values are 0.25, 0.75, 1.25, 1.75,
    2.5, 3.5 and 5.  A value exactly on a midpoint goes to the neighbour whose
    code is even, so the comparison is strict where the lower code is even and
    non-strict where the upper code is even.  Values above 5 saturate to 6.
    """
    v = f32(v)
    code = ((v > F32(0.25)).astype(np.uint8)
            + (v >= F32(0.75))
            + (v > F32(1.25))
            + (v >= F32(1.75))
            + (v > F32(2.5))
            + (v >= F32(3.5))
            + (v > F32(5.0)))
    return code.astype(np.uint8)


def e2m1_decode(nibble) -> np.ndarray:
    """4-bit code (sign in bit 3) -> float32 value."""
    n = np.asarray(nibble, dtype=np.uint8)
    mag = E2M1_VALUES[n & 7]
    return np.where(n & 8, -mag, mag).astype(np.float32)


# ----------------------------------------------------------------------------
# NF4 codebook
# ----------------------------------------------------------------------------
NF4_OUTER_PROBABILITY = 0.5 * ((1.0 - 1.0 / (2 * 15)) + (1.0 - 1.0 / (2 * 16)))


def nf4_codebook() -> np.ndarray:
    """The 16 NormalFloat levels c_0 < ... < c_15 as float32 (c_0=-1, c_7=0, c_15=1).

    Positive side: N(0,1) quantiles at 8 probabilities evenly spaced from the
    outer probability down towards 1/2 (1/2 itself excluded); negative side:
    the mirror of 7 quantiles spaced the same way; plus an exact zero.  All
    levels are divided by the largest magnitude, in float64, then rounded to
    float32.
    """
    from scipy.stats import norm

    p = NF4_OUTER_PROBABILITY
    pos = norm.ppf(np.linspace(p, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(p, 0.5, 8)[:-1])
    levels = np.sort(np.concatenate([neg, [0.0], pos]))
    levels = levels / np.max(np.abs(levels))
    return levels.astype(np.float32)


def nf4_midpoints(codebook=None) -> np.ndarray:
    """m_j = fl32((c_j + c_{j+1}) / 2) with the sum taken in float64, j = 0..14."""
    c = nf4_codebook() if codebook is None else np.asarray(codebook, dtype=np.float32)
    c64 = c.astype(np.float64)
    return ((c64[:-1] + c64[1:]) / 2.0).astype(np.float32)
