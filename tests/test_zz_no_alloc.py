"""The allocation-free quantizer entry point (bqm_quantize_nvfp4_noalloc) against
bqm_quantize_nvfp4 with a caller workspace: codes, block scales and s_dec bit for
bit, on two calls in a row (the second with fewer and smaller matrices, so a
running amax left over from the first call would show), in per-tensor mode with
the static scratch, with caller scales and in per-row mode."""
import pytest

import synth
from tests.gpu_util import gpu, log

pytestmark = pytest.mark.gpu


def _pair(x, mode=0, s_dec_in=None, fos=1):
    import torch
    import bit_quantized_moe_amd as bqm
    n, rows, cols = x.shape
    ref = bqm.alloc_qtensor(bqm.FMT_NVFP4, n, rows, cols, device=x.device, scale_mode=mode)
    got = bqm.alloc_qtensor(bqm.FMT_NVFP4, n, rows, cols, device=x.device, scale_mode=mode)
    wsb = bqm.bqm_quantize_nvfp4_workspace_size(n, rows, cols, mode)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    bqm.bqm_quantize_nvfp4(x, fos, s_dec_in, ref, ws)
    bqm.bqm_quantize_nvfp4_noalloc(x, fos, s_dec_in, got)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, what):
    import torch
    assert torch.equal(ref.codes, got.codes), f"{what}: codes"
    assert torch.equal(ref.scales, got.scales), f"{what}: scales"
    assert torch.equal(ref.s_dec.view(torch.int32), got.s_dec.view(torch.int32)), f"{what}: s_dec"


def test_noalloc_matches_workspace_entry_point_twice():
    dev = gpu()
    x1 = synth.normal((7, 96, 512), 0.5, (31, 1), device=dev, outliers=True)
    ref, got = _pair(x1)
    _same(ref, got, "first call")
    # fewer, smaller matrices with a smaller amax: the scratch must start from zero again
    x2 = synth.normal((3, 40, 272), 0.01, (31, 2), device=dev, outliers=False)
    ref2, got2 = _pair(x2)
    _same(ref2, got2, "second call")
    assert float(got2.s_dec.max()) < float(got.s_dec.min())
    for fos in (0, 2):
        _same(*_pair(x2, fos=fos), f"four_over_six={fos}")
    _same(*_pair(x2, s_dec_in=ref2.s_dec.clone()), "caller scales")
    _same(*_pair(x2, mode=1), "per-row")
    log("no-alloc quantizer matches the workspace entry point")
