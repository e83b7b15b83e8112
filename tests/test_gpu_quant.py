"""GPU parity of the quantizers, dequantizers, router and permutation (bit-exact)."""
import numpy as np
import pytest

from oracle import formats as fm
from oracle import quant as oq
from oracle import routing as orr
from tests.gpu_util import gpu, log, np_f32, np_u8
import synth

pytestmark = pytest.mark.gpu


def _bqm():
    import bit_quantized_moe_amd as bqm
    return bqm


def gpu_quant_nvfp4(x, fos=True, per_row=False, s_dec_in=None):
    import torch
    bqm = _bqm()
    n, rows, cols = x.shape
    mode = bqm.SCALE_PER_ROW if per_row else bqm.SCALE_PER_TENSOR
    q = bqm.alloc_qtensor(bqm.FMT_NVFP4, n, rows, cols, device=x.device, scale_mode=mode)
    wsb = bqm.bqm_quantize_nvfp4_workspace_size(n, rows, cols, mode)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    bqm.bqm_quantize_nvfp4(x, int(fos), s_dec_in, q, ws)
    return q


def check_nvfp4_against_oracle(x_dev, q, fos, per_row, s_dec_in=None, mats=None):
    n_mat = x_dev.shape[0]
    mats = range(n_mat) if mats is None else mats
    for m in mats:
        x = np_f32(x_dev[m:m + 1])
        sdi = None
        if s_dec_in is not None:
            sdi = np_f32(s_dec_in).reshape((n_mat, -1) if per_row else (-1,))[m:m + 1]
        ref = oq.quantize_nvfp4(x, four_over_six=fos, per_row=per_row, s_dec_in=sdi)
        got_c = np_u8(q.codes[m])
        got_s = np_u8(q.scales[m])
        if per_row:
            got_sd = np_f32(q.s_dec.view(n_mat, -1)[m])
        else:
            got_sd = np_f32(q.s_dec[m:m + 1])
        bad = np.nonzero(got_c != ref.codes[0])
        assert bad[0].size == 0, f"matrix {m}: {bad[0].size} code bytes differ, first at {bad[0][0]},{bad[1][0]}"
        assert (got_s == ref.scales[0]).all(), f"matrix {m}: scales differ"
        assert (got_sd.view(np.uint32) == ref.s_dec.reshape(-1).view(np.uint32)).all(), f"matrix {m}: s_dec"


@pytest.mark.parametrize("fos", [True, False])
@pytest.mark.parametrize("shape", [(3, 64, 256), (2, 37, 48), (1, 1, 16), (5, 130, 160)])
def test_nvfp4_per_tensor_bit_exact(shape, fos):
    dev = gpu()
    log(f"nvfp4 per-tensor {shape} fos={fos}")
    x = synth.normal(shape, 0.02, (90, shape[1], shape[2]), device="cpu", outliers=True).to(dev)
    q = gpu_quant_nvfp4(x, fos=fos)
    check_nvfp4_against_oracle(x, q, fos, per_row=False)


@pytest.mark.parametrize("shape", [(1, 64, 2048), (2, 33, 768), (1, 3, 6144)])
def test_nvfp4_per_row_bit_exact(shape):
    dev = gpu()
    log(f"nvfp4 per-row {shape}")
    x = synth.normal(shape, 1.0, (91, shape[1], shape[2]), device="cpu").to(dev)
    q = gpu_quant_nvfp4(x, fos=True, per_row=True)
    check_nvfp4_against_oracle(x, q, True, per_row=True)


def test_nvfp4_given_scale_and_edge_blocks():
    import torch
    dev = gpu()
    log("nvfp4 s_dec_in, zero blocks, worked example")
    x = synth.normal((2, 16, 64), 0.02, (92,), device="cpu", outliers=True)
    x[0, 3, 16:32] = 0.0
    x[1] = 0.0                                   # an all-zero matrix: s_dec = 1
    x[0, 5, :16] = -0.0
    x = x.to(dev)
    q = gpu_quant_nvfp4(x)
    check_nvfp4_against_oracle(x, q, True, per_row=False)
    sdi = torch.tensor([3e-4, 1.0], dtype=torch.float32, device=dev)
    q2 = gpu_quant_nvfp4(x, s_dec_in=sdi)
    check_nvfp4_against_oracle(x, q2, True, per_row=False, s_dec_in=sdi)
    # the GLM page's worked example, padded to one 16-block per row
    w = torch.zeros((1, 2, 16), dtype=torch.bfloat16)
    w[0, :, :3] = torch.tensor([[1, 2, 3], [4, 5, 6]], dtype=torch.bfloat16)
    q3 = gpu_quant_nvfp4(w.to(dev), fos=True)
    y = torch.empty((1, 2, 16), dtype=torch.bfloat16, device=dev)
    _bqm().bqm_dequantize(q3, y)
    assert np_f32(y)[0, :, :3].tolist() == [[1, 2, 3], [4.5, 4.5, 6]]


@pytest.mark.parametrize("per_row", [False, True])
def test_nvfp4_dequantize_bit_exact(per_row):
    import torch
    dev = gpu()
    x = synth.normal((3, 48, 128), 0.02, (93,), device="cpu", outliers=True).to(dev)
    q = gpu_quant_nvfp4(x, per_row=per_row)
    y = torch.empty_like(x)
    _bqm().bqm_dequantize(q, y)
    ref = oq.dequantize_nvfp4(oq.NVFP4Tensor(np_u8(q.codes), np_u8(q.scales),
                                             np_f32(q.s_dec).reshape((3, -1) if per_row else (-1,)),
                                             True, per_row))
    assert (np_f32(y).view(np.uint32) == ref.view(np.uint32)).all()


@pytest.mark.parametrize("per_row", [False, True])
def test_nvfp4_strict_four_over_six_bit_exact(per_row):
    """four_over_six = 2: the strict FP32 reference error for the 4/6 choice."""
    import torch
    dev = gpu()
    bqm = _bqm()
    shape = (3, 64, 256) if not per_row else (2, 33, 768)
    log(f"nvfp4 strict 4/6 {shape} per_row={per_row}")
    x = synth.normal(shape, 0.02 if not per_row else 1.0, (96, shape[1]), device="cpu", outliers=True).to(dev)
    n, rows, cols = shape
    mode = bqm.SCALE_PER_ROW if per_row else bqm.SCALE_PER_TENSOR
    q = bqm.alloc_qtensor(bqm.FMT_NVFP4, n, rows, cols, device=dev, scale_mode=mode)
    ws = torch.empty(max(bqm.bqm_quantize_nvfp4_workspace_size(n, rows, cols, mode), 16), dtype=torch.uint8, device=dev)
    bqm.bqm_quantize_nvfp4(x, 2, None, q, ws)
    for m in range(n):
        ref = oq.quantize_nvfp4(np_f32(x[m:m + 1]), four_over_six=True, per_row=per_row, strict=True)
        assert (np_u8(q.codes[m]) == ref.codes[0]).all(), f"matrix {m}: codes"
        assert (np_u8(q.scales[m]) == ref.scales[0]).all(), f"matrix {m}: scales"
        got_sd = np_f32(q.s_dec.view(n, -1)[m]) if per_row else np_f32(q.s_dec[m:m + 1])
        assert (got_sd.view(np.uint32) == ref.s_dec.reshape(-1).view(np.uint32)).all()
    assert q.four_over_six == 2


@pytest.mark.parametrize("fos", [True, False])
def test_nvfp4_block_scales_over_the_e4m3_range(fos):
    """Block scales E4M3(t/6) and E4M3(t/4) for every bf16 block maximum t in [2^-30, 2^13]:
    with a given s_dec of 1 the target is x itself, so this covers the E4M3 subnormals, every
    rounding boundary between E4M3 values and the saturation at 448 (t/6 > 448 above 2688)."""
    import torch
    dev = gpu()
    log(f"nvfp4 block scales over the E4M3 range, fos={fos}")
    bits = np.arange(0x3080, 0x4600, dtype=np.uint32)          # bf16 patterns 2^-30 .. 2^13 (exclusive)
    t = fm.bf16_bits_to_f32(bits.astype(np.uint16))
    x = np.zeros((t.size, 16), dtype=np.float32)
    x[:, 0] = t
    x[:, 5] = fm.bf16_round(-t * np.float32(0.3))
    x[:, 11] = fm.bf16_round(t * np.float32(0.55))
    x = x.reshape(1, t.size, 16)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.float().numpy(), x)
    sdi = torch.ones(1, dtype=torch.float32, device=dev)
    q = gpu_quant_nvfp4(xt.to(dev), fos=fos, s_dec_in=sdi)
    check_nvfp4_against_oracle(xt.to(dev), q, fos, per_row=False, s_dec_in=sdi)


@pytest.mark.parametrize("shape", [(2, 64, 256), (3, 5, 64), (1, 130, 192)])
def test_nf4_quantize_dequantize_bit_exact(shape):
    import torch
    dev = gpu()
    bqm = _bqm()
    log(f"nf4 {shape}")
    x = synth.normal(shape, 0.02, (94, shape[1]), device="cpu", outliers=True)
    x[0, 0, :64] = 0.0
    x = x.to(dev)
    q = bqm.alloc_qtensor(bqm.FMT_NF4, *shape, device=dev)
    bqm.bqm_quantize_nf4(x, q)
    ref = oq.quantize_nf4(np_f32(x))
    assert (np_u8(q.codes) == ref.codes).all()
    assert (np_f32(q.scales) == ref.absmax).all()
    y = torch.empty_like(x)
    bqm.bqm_dequantize(q, y)
    assert (np_f32(y).view(np.uint32) == oq.dequantize_nf4(ref).view(np.uint32)).all()


def _check_nested(q_plain, n, x_host, mats=None):
    """The nested stack n (from bqm_nf4_nest of q_plain) against the oracle's nesting
    of its own NF4 quantization of x_host, matrix by matrix, bit for bit."""
    for m in (range(x_host.shape[0]) if mats is None else mats):
        ref = oq.nest_absmax(oq.quantize_nf4(x_host[m:m + 1]))
        sd = np_f32(n.s_dec[m])
        assert sd[0].view(np.uint32) == ref.offset[0].view(np.uint32), f"matrix {m}: offset"
        assert (sd[1:].view(np.uint32) == ref.group_scale[0].view(np.uint32)).all(), f"matrix {m}: group scales"
        got = np_u8(n.scales[m])
        bad = np.nonzero(got != ref.absmax_q[0])
        assert bad[0].size == 0, f"matrix {m}: {bad[0].size} nested codes differ"
        assert (np_u8(n.codes[m]) == ref.codes[0]).all(), f"matrix {m}: codes"


@pytest.mark.parametrize("shape", [(3, 7, 640), (2, 96, 512), (1, 1, 64), (2, 300, 128)])
def test_nf4_nested_absmax_bit_exact(shape):
    # 70, 768, 1 and 600 blocks per matrix: one ragged group, whole groups, one
    # block, and a ragged third group; matrix 0 has a zero block, and a constant-
    # absmax matrix (every block scaled to the same largest value) where available
    import torch
    dev = gpu()
    bqm = _bqm()
    log(f"nf4 nested {shape}")
    x = synth.normal(shape, 0.02, (95, shape[1]), device="cpu", outliers=True)
    x[0, 0, :64] = 0.0
    if shape[0] > 1:
        xb = x[1].reshape(-1, 64).float()
        xb[:, 0] = 0.5                               # absmax 0.5 in every block
        x[1] = xb.clamp(-0.5, 0.5).to(torch.bfloat16).reshape(x[1].shape)
    xh = np_f32(x)
    x = x.to(dev)
    q = bqm.alloc_qtensor(bqm.FMT_NF4, *shape, device=dev)
    bqm.bqm_quantize_nf4(x, q)
    n = bqm.alloc_qtensor(bqm.FMT_NF4, *shape, device=dev, nested=1)
    bqm.bqm_nf4_nest(q, n)                           # separate codes buffer: copied
    torch.cuda.synchronize()
    _check_nested(q, n, xh)
    if shape[0] > 1:
        assert (np_f32(n.s_dec[1])[1:] == 0).all()   # constant absmax: d = 0 everywhere
    y = torch.empty_like(x)
    bqm.bqm_dequantize(n, y)
    ref = oq.dequantize_nf4_nested(oq.nest_absmax(oq.quantize_nf4(xh)))
    assert (np_f32(y).view(np.uint32) == ref.view(np.uint32)).all()
    # nesting twice gives the same bits (the offset comes from the exact sum)
    n2 = bqm.alloc_qtensor(bqm.FMT_NF4, *shape, device=dev, nested=1)
    n2.codes = q.codes
    bqm.bqm_nf4_nest(q, n2)
    assert torch.equal(n2.scales, n.scales) and torch.equal(n2.s_dec, n.s_dec)


def test_nf4_nested_offset_is_the_rounded_exact_sum():
    """The nesting offset is fl32(fl64(exact sum) / nb): absmax 2^70, 2^46 and three of
    2^16 in a matrix of 4096 blocks (every other block zero).  The exact sum rounds to
    2^70 + 2^46 + 2^18, and divided by 2^12 it lies just above the FP32 midpoint
    2^58 + 2^34, so the offset is 2^58 + 2^35; adding 2^16 to 2^70 + 2^46 one at a time
    in FP64 loses each of them and ends on the midpoint itself, which rounds to 2^58.
    A second matrix spreads absmax over 2^-120 .. 2^120 (random blocks)."""
    import torch
    dev = gpu()
    bqm = _bqm()
    shape = (2, 64, 4096)
    log(f"nf4 nested offset, exact sum {shape}")
    x = torch.zeros(shape, dtype=torch.float32)
    for blk, v in ((0, 2.0 ** 70), (1, 2.0 ** 46), (2, 2.0 ** 16), (3, 2.0 ** 16), (4, 2.0 ** 16)):
        x[0].view(-1)[64 * blk] = v
    rng = np.random.default_rng(123)
    e = rng.integers(-120, 121, size=shape[1] * shape[2] // 64)
    mag = np.ldexp(1.0 + rng.integers(0, 128, size=e.size) / 128.0, e)
    x[1].view(-1, 64)[:, 0] = torch.from_numpy(mag.astype(np.float32))
    x = x.to(torch.bfloat16)
    xh = np_f32(x)
    off = oq.nest_absmax(oq.quantize_nf4(xh[0:1])).offset[0]
    assert off == np.float32(2.0 ** 58 + 2.0 ** 35)     # the oracle's own arithmetic
    xd = x.to(dev)
    q = bqm.alloc_qtensor(bqm.FMT_NF4, *shape, device=dev)
    bqm.bqm_quantize_nf4(xd, q)
    n = bqm.alloc_qtensor(bqm.FMT_NF4, *shape, device=dev, nested=1)
    bqm.bqm_nf4_nest(q, n)
    torch.cuda.synchronize()
    _check_nested(q, n, xh)
    y = torch.empty_like(xd)
    bqm.bqm_dequantize(n, y)
    ref = oq.dequantize_nf4_nested(oq.nest_absmax(oq.quantize_nf4(xh)))
    assert (np_f32(y).view(np.uint32) == ref.view(np.uint32)).all()


def test_nf4_nested_full_size_sampled():
    """Nested absmax of the full gate_up stack [256, 4096, 6144] (1536 groups per
    matrix); two matrices against the oracle, bit for bit."""
    import torch
    dev = gpu()
    bqm = _bqm()
    log("nested NF4 at full size: generating the gate_up stack on the device")
    wgu, wdn = synth.quantizer_stacks(device=dev)
    del wdn
    torch.cuda.empty_cache()
    q = bqm.alloc_qtensor(bqm.FMT_NF4, *wgu.shape, device=dev)
    bqm.bqm_quantize_nf4(wgu, q)
    n = bqm.alloc_qtensor(bqm.FMT_NF4, *wgu.shape, device=dev, nested=1)
    n.codes = q.codes
    bqm.bqm_nf4_nest(q, n)
    torch.cuda.synchronize()
    for m in (0, 201):
        log(f"  matrix {m}: oracle quantize + nest")
        ref = oq.nest_absmax(oq.quantize_nf4(np_f32(wgu[m:m + 1])))
        sd = np_f32(n.s_dec[m])
        assert sd[0].view(np.uint32) == ref.offset[0].view(np.uint32)
        assert (sd[1:].view(np.uint32) == ref.group_scale[0].view(np.uint32)).all()
        assert (np_u8(n.scales[m]) == ref.absmax_q[0]).all()
    del q, n, wgu
    torch.cuda.empty_cache()


def test_nf4_codes_at_midpoints_and_bucket_edges():
    """NF4 coding near its decision points: in blocks whose absmax is 1 (so x / absmax
    is x), every midpoint between two levels, its bf16 neighbours, every multiple of
    1/64 in [-1, 1] and their bf16 neighbours; the same blocks scaled by 2^-7, and by -3."""
    import torch
    dev = gpu()
    bqm = _bqm()
    mids = fm.nf4_midpoints().astype(np.float32)
    grid = (np.arange(-64, 65, dtype=np.float32) / 64.0).astype(np.float32)
    pts = np.concatenate([mids, grid]).astype(np.float32)
    b = fm.bf16_rne_bits(pts).astype(np.int64)
    vals = fm.bf16_bits_to_f32(np.concatenate([b - 1, b, b + 1]).astype(np.uint16))
    vals = vals[(np.abs(vals) <= 1.0) & ((vals == 0) | (np.abs(vals) >= 2.0 ** -60))]   # no bf16 subnormals
    per = 63                                        # the 64th element of each block is its absmax, 1
    nblk = -(-vals.size // per)
    v = np.zeros(nblk * per, dtype=np.float32)
    v[:vals.size] = vals
    blocks = np.concatenate([v.reshape(nblk, per), np.ones((nblk, 1), np.float32)], axis=1)
    # (the third copy, times -3, is rounded to bf16: near the decision points, not on them)
    x = np.concatenate([blocks, blocks * np.float32(2.0 ** -7), fm.bf16_round(-blocks * np.float32(3.0))], axis=0)
    x = x.reshape(1, -1, 64)
    log(f"nf4 decision points: {x.size} elements")
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.float().numpy(), x)    # every value is a bf16
    q = bqm.alloc_qtensor(bqm.FMT_NF4, *x.shape, device=dev)
    bqm.bqm_quantize_nf4(xt.to(dev), q)
    ref = oq.quantize_nf4(x)
    assert (np_u8(q.codes) == ref.codes).all()
    assert (np_f32(q.scales) == ref.absmax).all()


@pytest.mark.parametrize("shape,per_row", [((3, 64, 256), False), ((3, 37, 272), False), ((2, 37, 272), True),
                                           ((1, 1, 16), False), ((2, 1024, 1024), False)])
def test_nvfp4_dequantize_shapes(shape, per_row):
    """Dequantize when a matrix spans many workgroups, when a workgroup spans many rows,
    and with a total that is not a multiple of a workgroup's share."""
    import torch
    dev = gpu()
    log(f"nvfp4 dequantize {shape} per_row={per_row}")
    x = synth.normal(shape, 0.02, (95, shape[1], shape[2]), device="cpu", outliers=True).to(dev)
    q = gpu_quant_nvfp4(x, per_row=per_row)
    y = torch.empty_like(x)
    _bqm().bqm_dequantize(q, y)
    n = shape[0]
    ref = oq.dequantize_nvfp4(oq.NVFP4Tensor(np_u8(q.codes), np_u8(q.scales),
                                             np_f32(q.s_dec).reshape((n, -1) if per_row else (-1,)),
                                             True, per_row))
    assert (np_f32(y).view(np.uint32) == ref.view(np.uint32)).all()


# (the permutation ranks equal experts within each 64-pair group by lane: E = 16 with
# ties puts many equal experts in every group; E = 1000 is not a multiple of the
# 64-lane scan width; E = 1024 is the largest expert count, several 2048-pair chunks;
# up to 2048 routed pairs run the one-workgroup form, ties and E = 1024 included; the
# router keeps 1, 2, 4, 8 or 16 logits per lane: E = 1 .. 1024 covers each)
@pytest.mark.parametrize("T,E,k,kind", [(64, 8, 2, "normal"), (1000, 256, 8, "uniform"),
                                        (333, 128, 8, "ties"), (50, 64, 16, "zipf"), (1, 1, 1, "normal"),
                                        (5000, 16, 2, "ties"), (700, 1000, 3, "zipf"),
                                        (3000, 1024, 4, "uniform"), (300, 16, 4, "ties"),
                                        (200, 1024, 8, "uniform"), (256, 1000, 8, "zipf"),
                                        (400, 512, 6, "ties"), (20, 300, 2, "zipf"), (9, 65, 5, "ties")])
def test_route_and_permute_bit_exact(T, E, k, kind):
    import torch
    dev = gpu()
    bqm = _bqm()
    log(f"route/permute T={T} E={E} k={k} {kind}")
    rng = np.random.default_rng(T + E)
    if kind == "ties":
        lg = (rng.integers(-4, 4, size=(T, E)) * 0.25).astype(np.float32)
    elif kind == "zipf":
        lg = (rng.gumbel(size=(T, E)) - 1.1 * np.log(rng.permutation(E) + 1.0)).astype(np.float32)
        lg[:, :8] = -np.inf
    elif kind == "uniform":
        lg = rng.random((T, E), dtype=np.float32)
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    lgd = torch.from_numpy(lg).to(dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    bqm.bqm_route(lgd, T, E, k, 0, idx, w)
    ridx, rw = orr.route(lg, k)
    assert (idx.cpu().numpy() == ridx).all()
    assert np.allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-9)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(bqm.bqm_permute_workspace_size(T, E, k), 16), dtype=torch.uint8, device=dev)
    bqm.bqm_permute(idx, T, E, k, perm, inv, off, ws)
    p, iv, o = orr.permute(ridx, E)
    assert (perm.cpu().numpy() == p).all() and (inv.cpu().numpy() == iv).all()
    assert (off.cpu().numpy() == o).all()
    _, rwr = orr.route(lg, k, renorm=True)
    bqm.bqm_route(lgd, T, E, k, 1, idx, w)
    assert np.allclose(w.cpu().numpy(), rwr, rtol=2e-6, atol=1e-9)


def test_quantizer_full_size_sampled():
    """The quantizer workload at full size (gate_up [256,4096,6144], down [256,6144,2048]);
    sampled matrices are checked bit-exactly, every matrix against the closed-form s_dec."""
    import torch
    dev = gpu()
    bqm = _bqm()
    log("full-size quantizer: generating 19.3 GB of bf16 weights on the device")
    wgu, wdn = synth.quantizer_stacks(device=dev)
    for name, w, mats in (("gate_up", wgu, [0, 131, 255]), ("down", wdn, [7, 200])):
        q = gpu_quant_nvfp4(w, fos=True)
        torch.cuda.synchronize()
        amax = w.view(w.shape[0], -1).abs().amax(dim=1).float().cpu()
        s_ref = amax / 1536.0                      # IEEE division on the host
        assert torch.equal(q.s_dec.cpu(), s_ref), name
        log(f"  {name}: s_dec closed form ok; checking matrices {mats} against the oracle")
        check_nvfp4_against_oracle(w, q, True, per_row=False, mats=mats)
        # DQ(Q(DQ(Q(W)))) == DQ(Q(W)) with the scale held fixed, on the whole stack
        y = torch.empty_like(w)
        bqm.bqm_dequantize(q, y)
        q2 = gpu_quant_nvfp4(y, fos=True, s_dec_in=q.s_dec)
        y2 = torch.empty_like(w)
        bqm.bqm_dequantize(q2, y2)
        assert torch.equal(y2.view(torch.int16), y.view(torch.int16)), name
        log(f"  {name}: round trip idempotent")
        del y, y2, q2, q
        torch.cuda.empty_cache()
