"""NVFP4 (with Four-Over-Six) and NF4 block quantization, step by step.

Test infrastructure (see the package docstring).

NVFP4 follows "The 4-bitter Lesson: Balancing Stability and Performance in
NVFP4 RL": section "Method" (16-value blocks, one E4M3 scale per block, one FP32
scale per tensor, or per token for activations, computed across the hidden
dimension) and section "Four-Over-Six for RL Weights and Activations" (the
target is scaled down once by the inverse of amax / (E2M1_MAX * M); a second
candidate block scale uses amax/4 instead of amax/6; the blockwise squared
error, accumulated in FP32, picks the lower-error candidate).  Blocks are 16
consecutive elements along the last axis, the rowwise copy of "Getting GLM-5.2
NVFP4 Post-Training off the ground", section "Why can't we just transpose the
one copy?"; codes are packed two per byte (same page, the paragraph after).

Readings taken where the pages are silent:
* M (E4M3_4OVER6_MAX, named but never given a value) is 256 with 4/6 on: the
  largest power of two that keeps the tensor-max block's scale-to-4 candidate
  (6M/4) inside E4M3's 448.  With 4/6 off, M is 448.
* Everything rounds to nearest even; E4M3 and E2M1 saturate at their largest
  finite value.  The block scale is fl(t/k) rounded to E4M3, then the scaled
  block is multiplied by the FP32 reciprocal of that scale.
* The error of a candidate is sum_i fl(d_i * d_i), d_i = fl(y_i - q_i * sb),
  added in FP32 in element order 0..15.  Ties keep the scale-to-6 candidate.
* A zero code keeps the sign of its input; element 2j is the low nibble of byte j.
* Per-tensor means one 2-D expert slice: gate and up of one expert share one
  scale.

NF4 follows "nf4moe - QLoRA for a 743B Fused-MoE", section "The fix:
dequant-on-forward for routed experts" (blocksize 64, absmax per block): the
block is divided by its FP32 absmax (multiplied by the FP32 reciprocal) and each
element takes the nearest codebook level, ties going to the lower level.

Nested absmax (the same page names bnb's quant state as "absmax, nested code",
section "The fix: dequant-on-forward for routed experts"; it says nothing more,
so this follows the published
QLoRA double quantization): the FP32 absmax of one matrix, in row-major block
order, has its mean subtracted (offset = the exactly rounded sum over the block
count, in float64, rounded to FP32); each group of 256 consecutive blocks gets
s2 = fl(max|d| / 448) and the codes e4m3(fl(d / s2)), d = fl(absmax - offset),
E4M3 (OCP, round to nearest even, saturating, the sign bit set for d < 0)
standing for the 8-bit float.  A group with max|d| = 0 has s2 = 0 and codes 0.  The NF4 codes themselves come
from the exact absmax; dequantization uses absmax' = fl(fl(e4m3 * s2) + offset).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as fm

F32 = np.float32
M_4OVER6 = 256.0
M_PLAIN = 448.0
BLOCK = 16
NF4_BLOCK = 64


@dataclass
class NVFP4Tensor:
    codes: np.ndarray    # uint8 [..., C/2]
    scales: np.ndarray   # uint8 E4M3 bits [..., C/16]
    s_dec: np.ndarray    # float32: [n_mat] (per tensor) or [n_mat, rows] (per row)
    four_over_six: bool
    per_row: bool


@dataclass
class NF4Tensor:
    codes: np.ndarray    # uint8 [..., C/2]
    absmax: np.ndarray   # float32 [..., C/64]


@dataclass
class NF4Nested:
    codes: np.ndarray        # uint8 [n_mat, rows, C/2], as in the plain tensor
    absmax_q: np.ndarray     # uint8 E4M3 bits [n_mat, rows, C/64]
    group_scale: np.ndarray  # float32 [n_mat, G]: s2 of each 256-block group, G = ceil(rows C / 64 / 256)
    offset: np.ndarray       # float32 [n_mat]: the mean of the matrix's absmax


def global_decode_scale(amax, four_over_six: bool) -> tuple[np.ndarray, np.ndarray]:
    """s_dec = fl(A / fl(6*M)), s_enc = fl(1/s_dec); A = 0 gives (1, 1)."""
    m = M_4OVER6 if four_over_six else M_PLAIN
    denom = F32(6.0) * F32(m)                      # exact: 1536 or 2688
    a = fm.f32(amax)
    s_dec = np.where(a > 0, a / denom, F32(1.0)).astype(np.float32)
    s_enc = (F32(1.0) / s_dec).astype(np.float32)
    return s_dec, s_enc


def _quantize_blocks(y: np.ndarray, four_over_six: bool, strict=None):
    """Quantize already-scaled blocks y [nb, 16] (float32).

    strict = (x [nb,16], s_dec [nb]) selects the strict FP32 reference error of the
    4-bitter page (section "Four-Over-Six for RL Weights and Activations"): each
    candidate is scaled back up, fl(fl(q*sb) * s_dec), and compared with the original
    x; otherwise the error is taken in the scaled domain against y (the fast path that
    scales the target down once).  Returns (magnitude codes [nb,16] uint8, scale bits
    [nb] uint8).
    """
    ay = np.abs(y)
    t = ay.max(axis=1)                                    # block amax of the scaled target
    cands = (6.0, 4.0) if four_over_six else (6.0,)
    results = []
    for k in cands:
        sb_bits = fm.e4m3_rne_satfinite((t / F32(k)).astype(np.float32))
        sb = fm.e4m3_decode(sb_bits)
        r = np.where(sb > 0, F32(1.0) / np.where(sb > 0, sb, F32(1.0)), F32(0.0)).astype(np.float32)
        v = (ay * r[:, None]).astype(np.float32)
        mag = fm.e2m1_mag_code(v)
        qs = (fm.E2M1_VALUES[mag] * sb[:, None]).astype(np.float32)   # exact
        if strict is None:
            d = (ay - qs).astype(np.float32)
        else:
            ax, sdec = strict
            up = (qs * sdec[:, None]).astype(np.float32)                # one rounding
            d = (np.abs(ax) - up).astype(np.float32)
        dd = (d * d).astype(np.float32)
        err = np.zeros(y.shape[0], dtype=np.float32)
        for i in range(BLOCK):                              # sequential FP32 sum
            err = (err + dd[:, i]).astype(np.float32)
        results.append((mag, sb_bits, err))
    mag, sb_bits, err6 = results[0]
    if four_over_six:
        mag4, sb4, err4 = results[1]
        pick4 = err4 < err6
        mag = np.where(pick4[:, None], mag4, mag)
        sb_bits = np.where(pick4, sb4, sb_bits)
    return mag.astype(np.uint8), sb_bits.astype(np.uint8)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[..., C] nibbles -> [..., C/2] bytes, element 2j in the low nibble."""
    nib = nib.astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _quantize_rows_with_scale(x: np.ndarray, s_enc_rows: np.ndarray, four_over_six: bool, s_dec_rows=None):
    """x [rows, C] float32, s_enc per row [rows] -> (codes [rows,C/2], scales [rows,C/16]).
    s_dec_rows (per row) given: the strict FP32 4/6 error."""
    rows, C = x.shape
    y = (x * s_enc_rows[:, None]).astype(np.float32)
    yb = y.reshape(rows * (C // BLOCK), BLOCK)
    strict = None
    if s_dec_rows is not None:
        strict = (x.reshape(-1, BLOCK), np.repeat(fm.f32(s_dec_rows), C // BLOCK))
    mag, sb = _quantize_blocks(yb, four_over_six, strict)
    sign = np.signbit(x.reshape(-1, BLOCK)).astype(np.uint8) << 3
    nib = (mag | sign).reshape(rows, C)
    return pack_nibbles(nib), sb.reshape(rows, C // BLOCK)


def quantize_nvfp4(x, four_over_six: bool = True, per_row: bool = False,
                   s_dec_in=None, strict: bool = False) -> NVFP4Tensor:
    """Rowwise NVFP4 quantization of a stack x [n_mat, rows, C] (bf16 values as float32).

    per_row=False: one FP32 scale per 2-D matrix (weights).  per_row=True: one
    per row (per-token activation scales).  s_dec_in, if given, replaces the
    amax-derived decode scale ([n_mat] or [n_mat, rows]).  strict: the 4/6 choice
    uses the strict FP32 reference error (candidates scaled back up, compared with
    x) instead of the scaled-domain one; codes and candidate scales are the same.
    """
    x = fm.f32(x)
    if x.ndim == 2:
        x = x[None]
    n_mat, rows, C = x.shape
    if C % BLOCK:
        raise ValueError("columns must be a multiple of 16")
    if per_row:
        amax = np.abs(x).max(axis=2)                       # [n_mat, rows]
    else:
        amax = np.abs(x).reshape(n_mat, -1).max(axis=1)    # [n_mat]
    if s_dec_in is None:
        s_dec, s_enc = global_decode_scale(amax, four_over_six)
    else:
        s_dec = fm.f32(s_dec_in).reshape(amax.shape)
        s_enc = (F32(1.0) / s_dec).astype(np.float32)
    codes = np.empty((n_mat, rows, C // 2), dtype=np.uint8)
    scales = np.empty((n_mat, rows, C // BLOCK), dtype=np.uint8)
    for e in range(n_mat):
        se = s_enc[e] if per_row else np.full(rows, s_enc[e], dtype=np.float32)
        sd = None
        if strict and four_over_six:
            sd = s_dec[e] if per_row else np.full(rows, s_dec[e], dtype=np.float32)
        codes[e], scales[e] = _quantize_rows_with_scale(x[e], se, four_over_six, sd)
    return NVFP4Tensor(codes, scales, s_dec.astype(np.float32), four_over_six, per_row)


def nvfp4_block_values(q: NVFP4Tensor) -> np.ndarray:
    """val(q) * sb for every element (exact in float32): [n_mat, rows, C]."""
    nib = unpack_nibbles(q.codes)
    vals = fm.e2m1_decode(nib)
    sb = fm.e4m3_decode(q.scales)
    return (vals * np.repeat(sb, BLOCK, axis=-1)).astype(np.float32)


def dequantize_nvfp4(q: NVFP4Tensor) -> np.ndarray:
    """Round-trip output: bf16(fl(fl(val*sb) * s_dec)), returned as float32 values."""
    vs = nvfp4_block_values(q)
    if q.per_row:
        s = q.s_dec[:, :, None]
    else:
        s = q.s_dec[:, None, None]
    return fm.bf16_round((vs * s).astype(np.float32))


def dequantize_nvfp4_exact(q: NVFP4Tensor) -> np.ndarray:
    """GEMM operand: the exact value val*sb*s_dec in float64 (no rounding)."""
    vs = nvfp4_block_values(q).astype(np.float64)
    s = q.s_dec.astype(np.float64)
    s = s[:, :, None] if q.per_row else s[:, None, None]
    return vs * s


# ----------------------------------------------------------------------------
# NF4
# ----------------------------------------------------------------------------
def quantize_nf4(x, codebook=None) -> NF4Tensor:
    """NF4 quantization of x [n_mat, rows, C] (C % 64 == 0), blocks along the last axis."""
    x = fm.f32(x)
    if x.ndim == 2:
        x = x[None]
    n_mat, rows, C = x.shape
    if C % NF4_BLOCK:
        raise ValueError("columns must be a multiple of 64")
    mids = fm.nf4_midpoints(codebook)
    xb = x.reshape(-1, NF4_BLOCK)
    a = np.abs(xb).max(axis=1).astype(np.float32)
    r = np.where(a > 0, F32(1.0) / np.where(a > 0, a, F32(1.0)), F32(0.0)).astype(np.float32)
    xn = (xb * r[:, None]).astype(np.float32)
    code = np.zeros(xn.shape, dtype=np.uint8)
    for m in mids:                                   # count midpoints strictly below
        code += (xn > m).astype(np.uint8)
    codes = pack_nibbles(code.reshape(n_mat, rows, C))
    return NF4Tensor(codes, a.reshape(n_mat, rows, C // NF4_BLOCK))


def nf4_values_f32(q: NF4Tensor, codebook=None) -> np.ndarray:
    """fl32(c[code] * absmax) per element."""
    c = fm.nf4_codebook() if codebook is None else np.asarray(codebook, dtype=np.float32)
    nib = unpack_nibbles(q.codes)
    a = np.repeat(q.absmax, NF4_BLOCK, axis=-1)
    return (c[nib] * a).astype(np.float32)


def dequantize_nf4(q: NF4Tensor, codebook=None) -> np.ndarray:
    """bf16(fl32(c[code] * absmax)) as float32 values; also the GEMM operand."""
    return fm.bf16_round(nf4_values_f32(q, codebook))


NEST_GROUP = 256
E4M3_MAX = 448.0


def nest_absmax(q: NF4Tensor) -> NF4Nested:
    """Double quantization of the FP32 absmax, one matrix (leading index) at a time."""
    import math
    a = fm.f32(q.absmax)
    n_mat = a.shape[0]
    flat = a.reshape(n_mat, -1)
    nb = flat.shape[1]
    G = -(-nb // NEST_GROUP)
    codes = np.zeros(flat.shape, dtype=np.uint8)
    s2 = np.zeros((n_mat, G), dtype=np.float32)
    offset = np.zeros(n_mat, dtype=np.float32)
    for m in range(n_mat):
        offset[m] = np.float32(math.fsum(float(v) for v in flat[m]) / nb)
        d = (flat[m] - offset[m]).astype(np.float32)
        for g in range(G):
            dg = d[g * NEST_GROUP:(g + 1) * NEST_GROUP]
            t = np.abs(dg).max()
            sc = np.float32(t / F32(E4M3_MAX))
            s2[m, g] = sc
            if sc > 0:
                y = (dg / sc).astype(np.float32)
                mag = fm.e4m3_rne_satfinite(np.abs(y)).astype(np.uint8)
                codes[m, g * NEST_GROUP:(g + 1) * NEST_GROUP] = mag | np.where(y < 0, 0x80, 0).astype(np.uint8)
    return NF4Nested(q.codes, codes.reshape(a.shape), s2, offset)


def unnest_absmax(n: NF4Nested) -> np.ndarray:
    """absmax' = fl(fl(e4m3 * s2) + offset), float32 [n_mat, rows, C/64]."""
    n_mat = n.absmax_q.shape[0]
    flat = n.absmax_q.reshape(n_mat, -1)
    g = np.arange(flat.shape[1]) // NEST_GROUP
    v = fm.e4m3_decode(flat).astype(np.float32)
    prod = (v * n.group_scale[:, g]).astype(np.float32)
    return (prod + n.offset[:, None]).astype(np.float32).reshape(n.absmax_q.shape)


def dequantize_nf4_nested(n: NF4Nested, codebook=None) -> np.ndarray:
    """bf16(fl32(c[code] * absmax')) as float32 values; also the GEMM operand."""
    return dequantize_nf4(NF4Tensor(n.codes, unnest_absmax(n)), codebook)


def nf4_nested_bytes(n_elements: int, n_mat: int, rows_cols_per_mat: int) -> int:
    """Codes, one byte per 64 elements, and per matrix the offset plus one FP32 per 256 blocks."""
    groups = -(-(rows_cols_per_mat // NF4_BLOCK) // NEST_GROUP)
    return n_elements // 2 + n_elements // 64 + 4 * n_mat * (1 + groups)


def nvfp4_bytes(n_elements: int, n_mat: int) -> int:
    """Storage of one rowwise NVFP4 copy: 4-bit codes, one byte per 16, 4 bytes per matrix."""
    return n_elements // 2 + n_elements // 16 + 4 * n_mat


def nf4_bytes(n_elements: int) -> int:
    return n_elements // 2 + 4 * (n_elements // 64)
