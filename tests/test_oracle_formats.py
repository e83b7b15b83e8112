"""Pins of the oracle's number formats against brute force and library conversions."""
import numpy as np
import pytest
import torch

from oracle import formats as fm

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _neighbourhood_patterns(centers, half_width):
    c = np.asarray(centers, dtype=np.float32).view(np.uint32).astype(np.int64)
    offs = np.arange(-half_width, half_width + 1, dtype=np.int64)
    p = (c[:, None] + offs[None, :]).reshape(-1)
    p = p[(p >= 0)]
    return np.unique(p).astype(np.uint32).view(np.float32)


def _brute_e2m1(v):
    """Nearest grid value in float64; on a tie (two neighbours, one even code) the even code wins."""
    v64 = v.astype(np.float64)
    d = np.abs(v64[:, None] - GRID[None, :])
    tie = d == d.min(axis=1, keepdims=True)
    codes = np.arange(8)[None, :]
    key = np.where(tie, codes % 2, 2)
    return np.argmin(key, axis=1)


def test_e2m1_ladder_neighbourhoods_and_sweep():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    v = _neighbourhood_patterns(list(GRID[1:]) + mids, 4096)
    v = v[(v >= 0) & (v < 8)]
    # a strided sweep over every float32 pattern in [0, 8)
    top = np.float32(8.0).view(np.uint32)
    sweep = np.arange(0, int(top), 257, dtype=np.uint64).astype(np.uint32).view(np.float32)
    allv = np.concatenate([v, sweep, np.float32([0.0, 6.0, 7.999999])])
    got = fm.e2m1_mag_code(allv)
    exp = _brute_e2m1(allv)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, (allv[bad[:5]], got[bad[:5]], exp[bad[:5]])


def test_e2m1_exact_ties_go_to_even_code():
    ties = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert fm.e2m1_mag_code(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert fm.e2m1_mag_code(np.float32([6.0, 7.0, 100.0, 1e30])).tolist() == [7, 7, 7, 7]


def test_e2m1_decode_grid():
    nib = np.arange(16, dtype=np.uint8)
    vals = fm.e2m1_decode(nib)
    assert vals[:8].tolist() == GRID.tolist()
    assert (vals[8:] == -GRID).all()
    assert np.signbit(vals[8])          # code 8 is -0


def _torch_e4m3_bits(v):
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_matches_torch_rne_below_464():
    grid = fm.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    v = _neighbourhood_patterns(np.concatenate([grid, mids, [2.0 ** -10]]), 64)
    v = v[(v >= 0) & (v <= 464)]
    top = np.float32(464.0).view(np.uint32)
    sweep = np.arange(0, int(top) + 1, 331, dtype=np.uint64).astype(np.uint32).view(np.float32)
    allv = np.concatenate([v, sweep]).astype(np.float32)
    got = fm.e4m3_rne_satfinite(allv)
    exp = _torch_e4m3_bits(allv)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, (allv[bad[:5]], got[bad[:5]], exp[bad[:5]])


def test_e4m3_saturates_and_special_points():
    got = fm.e4m3_rne_satfinite(np.float32([464.0, 464.0001, 480.0, 1e9, 2.0 ** -10, 2.0 ** -10 * 1.0001]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x00, 0x01]
    assert fm.e4m3_decode(np.uint8([0x7E]))[0] == 448.0
    assert fm.e4m3_decode(np.uint8([0x01]))[0] == 2.0 ** -9
    assert np.isnan(fm.e4m3_decode(np.uint8([0x7F]))[0])
    assert fm.e4m3_decode(np.uint8([0x7C]))[0] == 384.0


def test_e4m3_decode_encode_roundtrip_all_codes():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = fm.e4m3_decode(codes)
    assert (fm.e4m3_rne_satfinite(vals) == codes).all()
    assert (np.diff(vals) > 0).all()


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # include exact ties: low half 0x8000 with both parities of the kept lsb
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, 1.0, 3.3895314e38])])
    got = fm.bf16_rne_bits(v)
    exp = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (got == exp).all()


def test_nf4_codebook_construction_invariants():
    from scipy.stats import norm

    c = fm.nf4_codebook()
    assert c.dtype == np.float32 and c.size == 16
    assert (np.diff(c) > 0).all()
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8
    # each level is a normal quantile rescaled by the outermost one
    scale = norm.ppf(fm.NF4_OUTER_PROBABILITY)
    pos_p = norm.cdf(c[8:].astype(np.float64) * scale)
    neg_p = norm.cdf(-c[:7].astype(np.float64) * scale)
    assert np.allclose(np.diff(pos_p[::-1]), np.diff(pos_p[::-1]).mean(), atol=1e-6)
    assert np.allclose(np.diff(neg_p), np.diff(neg_p).mean(), atol=1e-6)
    # positive spacing: 8 steps from the outer probability to 1/2; negative: 7 steps
    assert np.isclose(pos_p[-1] - pos_p[-2], (fm.NF4_OUTER_PROBABILITY - 0.5) / 8, atol=1e-6)
    assert np.isclose(neg_p[0] - neg_p[1], (fm.NF4_OUTER_PROBABILITY - 0.5) / 7, atol=1e-6)
    m = fm.nf4_midpoints()
    assert m.size == 15 and (m[:7] < 0).all() and (m[7:] > 0).all()
