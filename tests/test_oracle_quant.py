"""Pins of the oracle's NVFP4 (Four-Over-Six) and NF4 quantizers.

Each test checks the oracle against something other than itself: the worked
example printed on the GLM-5.2 page (values derived by hand below from the
rules), exact rational arithmetic, brute-force nearest-value search, closed
forms and invariants that any correct implementation of the rules satisfies.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as fm
from oracle import quant as oq

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16_values(a):
    return fm.bf16_round(np.asarray(a, dtype=np.float32))


def _rand_weights(shape, seed, std=0.02, outliers=True):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape).astype(np.float32) * np.float32(std)
    if outliers:
        a = np.where(rng.random(shape) < 0.001, a * 20, a)
    return _bf16_values(a)


# ----------------------------------------------------------------------------
# the page's worked example
# ----------------------------------------------------------------------------
def _worked():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        g = json.load(f)
    W = np.zeros((2, 16), dtype=np.float32)
    W[:, :3] = np.array(g["W"], dtype=np.float32)
    return g, W


def test_worked_example_page_facts():
    g, W = _worked()
    # rowwise amaxes are the row scales the page names; the column block needs 4
    assert np.abs(W).max(axis=1).tolist() == g["row_scales"]
    col = np.array(g["column_block"], dtype=np.float32)
    assert np.abs(col).max() == g["column_scale_needed"]
    # no rowwise block scale equals the column's amax
    assert g["column_scale_needed"] not in g["row_scales"]


def test_worked_example_without_four_over_six():
    # A = 6, M = 448: s_dec = 6/2688 = 1/448, targets are x*448.
    # row 0: t = 1344, sb = E4M3(224) = 224, v = (2, 4, 6) -> exact, DQ = (1, 2, 3)
    # row 1: t = 2688, sb = 448, v = (4, 5, 6); 5 is the 4|6 tie -> even code (value 4)
    _, W = _worked()
    q = oq.quantize_nvfp4(W[None], four_over_six=False)
    sb = fm.e4m3_decode(q.scales[0, :, 0])
    assert sb.tolist() == [224.0, 448.0]
    vals = fm.e2m1_decode(oq.unpack_nibbles(q.codes[0]))[:, :3]
    assert vals.tolist() == [[2, 4, 6], [4, 4, 6]]
    dq = oq.dequantize_nvfp4(q)[0][:, :3]
    assert dq.tolist() == [[1, 2, 3], [4, 4, 6]]


def test_worked_example_with_four_over_six():
    # A = 6, M = 256: s_dec = 1/256 exactly, targets are x*256.
    # row 0: t = 768.  k=6: sb=128, v=(2,4,6), error 0.  k=4: sb=192,
    #        v=(1.33,2.67,4)->(1.5,3,4), q*sb=(288,576,768), error 32^2+64^2 -> keep 6.
    # row 1: t = 1536. k=6: sb=256, v=(4,5,6)->(4,4,6), error 256^2 = 65536.
    #        k=4: sb=384, v=(2.67,3.33,4)->(3,3,4), q*sb=(1152,1152,1536),
    #        error 128^2+128^2 = 32768 < 65536 -> pick 4; DQ = (4.5, 4.5, 6).
    _, W = _worked()
    q = oq.quantize_nvfp4(W[None], four_over_six=True)
    assert q.s_dec[0] == np.float32(1.0 / 256)
    sb = fm.e4m3_decode(q.scales[0, :, 0])
    assert sb.tolist() == [128.0, 384.0]
    assert q.scales[0, 1, 0] == 0x7C
    vals = fm.e2m1_decode(oq.unpack_nibbles(q.codes[0]))[:, :3]
    assert vals.tolist() == [[2, 4, 6], [3, 3, 4]]
    dq = oq.dequantize_nvfp4(q)[0][:, :3]
    assert dq.tolist() == [[1, 2, 3], [4.5, 4.5, 6]]
    # the padded zeros stay (+)0 codes
    assert (oq.unpack_nibbles(q.codes[0])[:, 3:] == 0).all()


def test_worked_example_columnwise_copy():
    # The page's column blocks {1,4}, {2,5}, {3,6} (amax 4, 5, 6) quantized as the rows of
    # W^T, targets x*256.  {256, 1024}: k=6 sb=E4M3(170.7)=176, v=(1.45,5.82)->(1.5,6),
    #   q*sb=(264,1056), error 8^2+32^2=1088; k=4 sb=256, v=(1,4), error 0 -> 4, DQ (1, 4).
    # {512, 1280}: k=6 sb=E4M3(213.3)=208, v=(2.46,6.15)->(2,6), q*sb=(416,1248), error
    #   96^2+32^2=10240; k=4 sb=320, v=(1.6,4)->(1.5,4), q*sb=(480,1280), error 1024 -> 4,
    #   DQ (1.875, 5).
    # {768, 1536}: k=6 sb=256, v=(3,6) exact; k=4 sb=384, v=(2,4) exact; the tie keeps 6.
    from oracle import moe as om
    g, W = _worked()
    Wt = np.zeros((16, 16), dtype=np.float32)    # W^T padded: the column blocks become 16-blocks
    Wt[:3, :2] = np.array(g["W"], dtype=np.float32).T
    q = oq.quantize_nvfp4(Wt[None], four_over_six=True)
    assert fm.e4m3_decode(q.scales[0, :3, 0]).tolist() == g["columnwise_block_scales"]
    Wp = np.zeros((16, 3), dtype=np.float32)     # W padded with zero rows (16-blocks run along rows)
    Wp[:2] = np.array(g["W"], dtype=np.float32)
    col = om.ColumnwiseExperts(lambda e: Wp).matrix(0)[:2]
    assert col.tolist() == g["columnwise_dq"]
    # the rowwise copy of the same W gives other values in the column {1, 4}
    dq_row = oq.dequantize_nvfp4(oq.quantize_nvfp4(W[None], four_over_six=True))[0][:, :3]
    assert dq_row[:, 0].tolist() == [1, 4.5] and col[:, 0].tolist() == [1, 4]


# ----------------------------------------------------------------------------
# exact rational arithmetic and brute force
# ----------------------------------------------------------------------------
def _exact_choice(y_row, sb6, sb4):
    """Exact-rational 4/6 choice: brute-force nearest E2M1 value of y/sb (ties to even code)."""
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    errs = []
    for sb in (sb6, sb4):
        sbf = Fraction(float(sb))
        e = Fraction(0)
        for y in y_row:
            ay = abs(Fraction(float(y)))
            if sbf == 0:
                q = Fraction(0)
            else:
                v = ay / sbf
                d = [abs(v - g) for g in grid]
                m = min(d)
                cands = [i for i, di in enumerate(d) if di == m]
                ci = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
                q = grid[ci]
            e += (ay - q * sbf) ** 2
        errs.append(e)
    return errs


def test_four_over_six_choice_agrees_with_exact_rationals():
    x = _rand_weights((1, 64, 256), seed=11)
    q = oq.quantize_nvfp4(x, four_over_six=True)
    s_enc = np.float32(1.0) / q.s_dec[0]
    y = (x[0] * s_enc).astype(np.float32).reshape(-1, 16)
    t = np.abs(y).max(axis=1)
    sb6 = fm.e4m3_decode(fm.e4m3_rne_satfinite((t / np.float32(6)).astype(np.float32)))
    sb4 = fm.e4m3_decode(fm.e4m3_rne_satfinite((t / np.float32(4)).astype(np.float32)))
    chosen = fm.e4m3_decode(q.scales[0].reshape(-1))
    disagree, near = 0, 0
    picks4 = 0
    for b in range(y.shape[0]):
        e6, e4 = _exact_choice(y[b], sb6[b], sb4[b])
        exact_pick4 = e4 < e6
        picks4 += exact_pick4
        got_pick4 = (chosen[b] == sb4[b]) and (sb4[b] != sb6[b])
        if exact_pick4 != got_pick4:
            disagree += 1
            # only near-ties may differ (FP32 rounding of the error terms)
            assert abs(float(e4 - e6)) <= 1e-4 * float(e6)
    assert disagree <= max(1, y.shape[0] // 500)
    # the second candidate actually wins a sizeable share of Gaussian blocks
    assert 0.05 < picks4 / y.shape[0] < 0.95


def _exact_strict_errors(x_row, y_row, sb6, sb4, s_dec):
    """Exact-rational strict errors: codes from the nearest E2M1 value of y/sb (ties to
    even), each candidate scaled back up by s_dec and compared with the original x."""
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    sd = Fraction(float(s_dec))
    errs = []
    for sb in (sb6, sb4):
        sbf = Fraction(float(sb))
        e = Fraction(0)
        for x, y in zip(x_row, y_row):
            ay = abs(Fraction(float(y)))
            q = Fraction(0)
            if sbf != 0:
                v = ay / sbf
                d = [abs(v - g) for g in grid]
                m = min(d)
                cands = [i for i, di in enumerate(d) if di == m]
                q = grid[[c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]]
            e += (abs(Fraction(float(x))) - q * sbf * sd) ** 2
        errs.append(e)
    return errs


def test_strict_four_over_six_choice_agrees_with_exact_rationals():
    # the strict FP32 reference error (4-bitter page, "Four-Over-Six for RL"): candidates
    # scaled back up by s_dec and compared with the original values
    x = _rand_weights((1, 32, 256), seed=21)
    q = oq.quantize_nvfp4(x, four_over_six=True, strict=True)
    s_dec = q.s_dec[0]
    y = (x[0] * (np.float32(1.0) / s_dec)).astype(np.float32).reshape(-1, 16)
    xb = x[0].reshape(-1, 16)
    t = np.abs(y).max(axis=1)
    sb6 = fm.e4m3_decode(fm.e4m3_rne_satfinite((t / np.float32(6)).astype(np.float32)))
    sb4 = fm.e4m3_decode(fm.e4m3_rne_satfinite((t / np.float32(4)).astype(np.float32)))
    chosen = fm.e4m3_decode(q.scales[0].reshape(-1))
    disagree = 0
    for b in range(y.shape[0]):
        e6, e4 = _exact_strict_errors(xb[b], y[b], sb6[b], sb4[b], s_dec)
        got_pick4 = (chosen[b] == sb4[b]) and (sb4[b] != sb6[b])
        if (e4 < e6) != got_pick4:
            disagree += 1
            assert abs(float(e4 - e6)) <= 1e-4 * float(e6)
    assert disagree <= max(1, y.shape[0] // 500)


def test_strict_and_scaled_four_over_six_agree_except_near_ties():
    # the two forms take the same codes and candidate scales and differ only in where
    # the squared error is measured; the page reports > 99.97% agreement between its
    # fast path and the strict reference
    x = _rand_weights((2, 256, 1024), seed=22)
    a = oq.quantize_nvfp4(x, four_over_six=True)
    b = oq.quantize_nvfp4(x, four_over_six=True, strict=True)
    assert (a.s_dec == b.s_dec).all()
    same = (a.scales == b.scales)
    frac = same.mean()
    assert frac >= 0.999, frac
    # where the scale agrees the codes agree too
    sa = np.repeat(same, 8, axis=-1)
    assert (a.codes[sa] == b.codes[sa]).all()
    # 4/6 off: the error form plays no part
    c = oq.quantize_nvfp4(x[:1, :32], four_over_six=False)
    d = oq.quantize_nvfp4(x[:1, :32], four_over_six=False, strict=True)
    assert (c.codes == d.codes).all() and (c.scales == d.scales).all()


def test_codes_are_nearest_grid_value_of_scaled_block():
    x = _rand_weights((2, 32, 128), seed=12)
    q = oq.quantize_nvfp4(x, four_over_six=True)
    vs = oq.nvfp4_block_values(q)                      # val*sb
    s_enc = (np.float32(1.0) / q.s_dec).astype(np.float32)
    y = (x * s_enc[:, None, None]).astype(np.float32)
    sb = np.repeat(fm.e4m3_decode(q.scales), 16, axis=-1).astype(np.float64)
    # |y - q*sb| <= half the local grid step of the chosen scale (+ saturation at 6*sb)
    v = np.abs(y).astype(np.float64) / sb
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    nearest = grid[np.abs(v[..., None] - grid).argmin(-1)]
    err_best = np.abs(v - nearest)
    err_got = np.abs(v - np.abs(vs) / sb)
    assert (err_got <= err_best + 1e-6).all()
    # signs follow the input
    assert (np.signbit(vs) == np.signbit(x)).all()


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_chosen_error_not_worse_than_scale_to_six():
    x = _rand_weights((3, 16, 64), seed=13)
    q46 = oq.quantize_nvfp4(x, four_over_six=True)
    s_enc = (np.float32(1.0) / q46.s_dec).astype(np.float32)
    y = (x * s_enc[:, None, None]).astype(np.float32).reshape(-1, 16)
    mag6, sb6 = oq._quantize_blocks(y, four_over_six=False)
    e6 = ((np.abs(y) - fm.E2M1_VALUES[mag6] * fm.e4m3_decode(sb6)[:, None]) ** 2).astype(np.float64).sum(1)
    vs = oq.nvfp4_block_values(q46).reshape(-1, 16).astype(np.float64)
    e = ((np.abs(y) - np.abs(vs)) ** 2).sum(1)
    assert (e <= e6 * (1 + 1e-5) + 1e-30).all()


def test_sign_symmetry():
    x = _rand_weights((2, 16, 64), seed=14)
    a = oq.quantize_nvfp4(x)
    b = oq.quantize_nvfp4(-x)
    assert (a.scales == b.scales).all() and (a.s_dec == b.s_dec).all()
    na, nb = oq.unpack_nibbles(a.codes), oq.unpack_nibbles(b.codes)
    assert ((na ^ nb) == 8).all()


@pytest.mark.parametrize("j", [-3, 2, 5])
def test_power_of_two_scaling(j):
    x = _rand_weights((2, 16, 64), seed=15)
    a = oq.quantize_nvfp4(x)
    b = oq.quantize_nvfp4((x * np.float32(2.0 ** j)).astype(np.float32))
    assert (a.codes == b.codes).all() and (a.scales == b.scales).all()
    assert (b.s_dec == (a.s_dec * np.float32(2.0 ** j))).all()


def test_permutation_within_block_permutes_codes():
    x = _rand_weights((1, 8, 64), seed=16)
    rng = np.random.default_rng(0)
    p = rng.permutation(16)
    xp = x.reshape(1, 8, 4, 16)[..., p].reshape(1, 8, 64)
    a, b = oq.quantize_nvfp4(x), oq.quantize_nvfp4(xp)
    na = oq.unpack_nibbles(a.codes).reshape(1, 8, 4, 16)[..., p]
    nb = oq.unpack_nibbles(b.codes).reshape(1, 8, 4, 16)
    assert (na == nb).all() and (a.scales == b.scales).all()


def test_zero_block_and_zero_tensor():
    x = _rand_weights((1, 4, 64), seed=17)
    x[0, 1, 16:32] = 0.0
    x[0, 2, 0:16] = -0.0
    q = oq.quantize_nvfp4(x)
    nib = oq.unpack_nibbles(q.codes)
    assert q.scales[0, 1, 1] == 0 and (nib[0, 1, 16:32] == 0).all()
    assert q.scales[0, 2, 0] == 0 and (nib[0, 2, 0:16] == 8).all()   # -0 keeps its sign
    z = oq.quantize_nvfp4(np.zeros((1, 2, 32), dtype=np.float32))
    assert z.s_dec[0] == 1.0 and (z.scales == 0).all() and (z.codes == 0).all()


def test_global_scale_closed_form_and_no_saturation():
    x = _rand_weights((4, 64, 128), seed=18)
    for fos, m in ((True, 256), (False, 448)):
        q = oq.quantize_nvfp4(x, four_over_six=fos)
        A = np.abs(x).reshape(4, -1).max(1)
        assert (q.s_dec == (A / np.float32(6 * m)).astype(np.float32)).all()
        # the tensor-max block's scale stays below E4M3's 448 (no saturation)
        assert fm.e4m3_decode(q.scales).max() < 448.0 or not fos


def test_round_trip_idempotent_with_fixed_scale():
    x = _rand_weights((3, 32, 128), seed=19)
    q1 = oq.quantize_nvfp4(x)
    d1 = oq.dequantize_nvfp4(q1)
    q2 = oq.quantize_nvfp4(d1, s_dec_in=q1.s_dec)
    d2 = oq.dequantize_nvfp4(q2)
    assert (d1 == d2).all()


def test_round_trip_error_bounded_by_grid_step():
    x = _rand_weights((2, 64, 128), seed=20)
    q = oq.quantize_nvfp4(x)
    dq = oq.dequantize_nvfp4(q)
    xb = x.reshape(-1, 16).astype(np.float64)
    db = dq.reshape(-1, 16).astype(np.float64)
    amax = np.abs(xb).max(1, keepdims=True)
    # E2M1 half-step at the top is 1 (of 6); E4M3 scale rounding adds 1/16; bf16 output rounding
    assert (np.abs(db - xb) <= amax * (1.0 / 6 + 1.0 / 16) * 1.02 + 1e-12).all()
    rel = np.linalg.norm(db - xb) / np.linalg.norm(xb)
    assert rel < 0.12


def test_per_row_mode_is_batch_invariant():
    x = _rand_weights((1, 24, 128), seed=21, std=1.0, outliers=False)
    full = oq.quantize_nvfp4(x, per_row=True)
    for r in (0, 7, 23):
        one = oq.quantize_nvfp4(x[:, r:r + 1], per_row=True)
        assert (one.codes[0, 0] == full.codes[0, r]).all()
        assert (one.scales[0, 0] == full.scales[0, r]).all()
        assert one.s_dec[0, 0] == full.s_dec[0, r]
    # a single-row matrix gives the same result in per-row and per-tensor mode
    a = oq.quantize_nvfp4(x[:, 5:6], per_row=True)
    b = oq.quantize_nvfp4(x[:, 5:6], per_row=False)
    assert (a.codes == b.codes).all() and a.s_dec.reshape(-1)[0] == b.s_dec[0]


def test_memory_closed_form():
    n_mat, rows, C = 4, 32, 256
    x = _rand_weights((n_mat, rows, C), seed=22)
    q = oq.quantize_nvfp4(x)
    N = n_mat * rows * C
    got = q.codes.nbytes + q.scales.nbytes + q.s_dec.nbytes
    assert got == oq.nvfp4_bytes(N, n_mat) == int(0.5625 * N) + 4 * n_mat
    qn = oq.quantize_nf4(x)
    assert qn.codes.nbytes + qn.absmax.nbytes == oq.nf4_bytes(N) == int(0.5625 * N)
    # 4.5 bits per weight: 16/4.5 = 3.56x smaller than bf16 (the nf4moe page's figure)
    assert round(2 * N / oq.nf4_bytes(N), 2) == 3.56


# ----------------------------------------------------------------------------
# NF4
# ----------------------------------------------------------------------------
def test_nf4_brute_force_nearest_level():
    x = _rand_weights((2, 16, 128), seed=23, std=1.0, outliers=False)
    q = oq.quantize_nf4(x)
    c = fm.nf4_codebook().astype(np.float64)
    a = np.repeat(q.absmax, 64, axis=-1).astype(np.float64)
    r = (np.float32(1.0) / np.repeat(q.absmax, 64, axis=-1)).astype(np.float32)
    xn = (x * r).astype(np.float32).astype(np.float64)
    d = np.abs(xn[..., None] - c)
    code = oq.unpack_nibbles(q.codes)
    best = d.min(-1)
    got = np.take_along_axis(d, code[..., None].astype(np.int64), -1)[..., 0]
    assert (got <= best + 1e-7).all()
    assert (q.absmax == np.abs(x).reshape(2, 16, 2, 64).max(-1)).all()


def test_nf4_absmax_element_decodes_exactly_and_zero_block():
    x = _rand_weights((1, 4, 128), seed=24, std=1.0, outliers=False)
    x[0, 3, 64:] = 0
    q = oq.quantize_nf4(x)
    dq = oq.dequantize_nf4(q)
    xb = x.reshape(-1, 64)
    db = dq.reshape(-1, 64)
    i = np.abs(xb).argmax(1)
    rows = np.arange(xb.shape[0])
    assert (db[rows, i] == xb[rows, i]).all()          # +-absmax is exact (bf16 input)
    nib = oq.unpack_nibbles(q.codes).reshape(-1, 64)
    assert (nib[-1] == 7).all() and (db[-1] == 0).all()


def test_nf4_midpoint_ties_go_to_lower_level():
    c = fm.nf4_codebook()
    m = fm.nf4_midpoints(c)
    # a block whose absmax is 1 and whose other entries sit exactly on midpoints
    blk = np.zeros(64, dtype=np.float32)
    blk[0] = 1.0
    blk[1:16] = m
    q = oq.quantize_nf4(blk[None, None, :])
    nib = oq.unpack_nibbles(q.codes)[0, 0]
    assert nib[0] == 15
    assert nib[1:16].tolist() == list(range(15))        # tie at m_j -> code j (lower)


def test_nf4_round_trip_error_small():
    x = _rand_weights((2, 64, 128), seed=25)
    dq = oq.dequantize_nf4(oq.quantize_nf4(x))
    rel = np.linalg.norm(dq - x) / np.linalg.norm(x)
    assert 0.03 < rel < 0.15


# ----------------------------------------------------------------------------
# NF4 with nested (double-quantized) absmax
# ----------------------------------------------------------------------------
def _nf4_plain(absmax_rows):
    """An NF4 tensor with the given absmax [n_mat, rows, nb] and zero codes."""
    a = np.asarray(absmax_rows, dtype=np.float32)
    n_mat, rows, nb = a.shape
    return oq.NF4Tensor(np.zeros((n_mat, rows, nb * 32), dtype=np.uint8), a)


def test_nested_absmax_hand_example():
    # two blocks with absmax 1 and 3: offset 2, d = -1, +1, s2 = fl(1/448), and the
    # codes are -448 and +448 (E4M3 0xFE / 0x7E); absmax' = 2 -/+ fl(448 fl(1/448))
    n = oq.nest_absmax(_nf4_plain([[[1.0, 3.0]]]))
    s2 = np.float32(np.float32(1.0) / np.float32(448.0))
    assert n.offset[0] == np.float32(2.0) and n.group_scale[0, 0] == s2
    assert list(n.absmax_q.reshape(-1)) == [0xFE, 0x7E]
    back = oq.unnest_absmax(n).reshape(-1)
    one = np.float32(np.float32(448.0) * s2)
    assert back[0] == np.float32(np.float32(2.0) - one) and back[1] == np.float32(np.float32(2.0) + one)


def test_nested_absmax_brute_force_and_bounds():
    import math
    from fractions import Fraction
    rng = np.random.default_rng(21)
    # 2 matrices of 7 x 100 blocks: 700 blocks, groups of 256, 256, 188 (ragged last)
    a = np.abs(rng.standard_normal((2, 7, 100)) * 0.03 + 0.05).astype(np.float32)
    a[1, 3, :] = 0.0                                   # zero blocks inside a group
    n = oq.nest_absmax(_nf4_plain(a))
    assert n.group_scale.shape == (2, 3)
    table = fm.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    back = oq.unnest_absmax(n)
    for m in range(2):
        flat = a[m].reshape(-1)
        exact = sum(Fraction(float(v)) for v in flat) / len(flat)
        off = n.offset[m]
        ulp = np.spacing(off)
        assert abs(Fraction(float(off)) - exact) <= Fraction(float(ulp))      # the mean, to one FP32 ulp
        d = (flat - off).astype(np.float32)
        for g in range(3):
            dg = d[g * 256:(g + 1) * 256]
            t = float(np.abs(dg).max())
            s2 = float(n.group_scale[m, g])
            assert s2 == float(np.float32(np.float32(t) / np.float32(448.0)))
            codes = n.absmax_q[m].reshape(-1)[g * 256:(g + 1) * 256]
            y = (dg / np.float32(s2)).astype(np.float64)
            for i in range(0, dg.size, 7):
                # nearest finite E4M3 value (NaN codes excluded), ties to the even code
                cand = [c for c in range(256) if c & 0x7F != 0x7F]
                dist = [abs(table[c] - min(y[i], 448.0) if y[i] >= 0 else abs(table[c] - max(y[i], -448.0))) for c in cand]
                best = min(dist)
                ok = [c for c, dd in zip(cand, dist) if dd == best]
                ok = [c for c in ok if (c & 0x80) == (0x80 if y[i] < 0 else 0)] or ok
                if len(ok) > 1:
                    ok = [c for c in ok if c % 2 == 0]
                assert codes[i] in ok, (m, g, i, y[i], codes[i], ok)
            # the E4M3 error bound: half a spacing, relative 2^-4 (normal) or 2^-10 absolute (subnormal)
            bm = back[m].reshape(-1)[g * 256:(g + 1) * 256].astype(np.float64)
            lim = s2 * np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 4 * np.spacing(np.float32(max(abs(off), t)))
            assert (np.abs(bm - flat[g * 256:(g + 1) * 256]) <= lim).all()
    del math


def test_nested_absmax_constant_and_zero_matrices():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((1, 16, 256)) * 0.1).astype(np.float32)
    q = oq.quantize_nf4(x)
    const = oq.NF4Tensor(q.codes, np.full_like(q.absmax, np.float32(0.3125)))
    n = oq.nest_absmax(const)
    assert (n.group_scale == 0).all() and (n.absmax_q == 0).all()
    assert (oq.unnest_absmax(n) == const.absmax).all()
    assert (oq.dequantize_nf4_nested(n) == oq.dequantize_nf4(const)).all()
    z = oq.quantize_nf4(np.zeros((1, 8, 128), np.float32))
    nz = oq.nest_absmax(z)
    assert (oq.dequantize_nf4_nested(nz) == 0).all() and nz.offset[0] == 0


def test_nested_absmax_storage_and_error():
    # storage: 4 + 8/64 + 32 / (64 * 256) bits per weight plus one FP32 per matrix
    # (QLoRA's 0.127 bits of quantization constants per weight, from 0.5)
    E, H, I = 256, 6144, 2048
    n_el = E * 2 * I * H + E * H * I
    b = oq.nf4_nested_bytes(E * 2 * I * H, E, 2 * I * H) + oq.nf4_nested_bytes(E * H * I, E, H * I)
    const_bits = 8 * b / n_el - 4
    assert abs(const_bits - (0.125 + 32 / (64 * 256))) < 1e-4
    assert 8 * (oq.nf4_bytes(n_el)) / n_el - 4 == 0.5
    # on N(0, 0.02) weights with outliers: absmax' is off by at most half an E4M3
    # spacing of the largest |d| of a group, 2^-4 of it, and |d| <= max absmax
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((2, 128, 512)) * 0.02).astype(np.float32)
    w[rng.random(w.shape) < 0.001] *= 20
    q = oq.quantize_nf4(w)
    n = oq.nest_absmax(q)
    err = np.abs(oq.unnest_absmax(n) - q.absmax).max() / q.absmax.max()
    assert 0 < err <= 2.0 ** -4
