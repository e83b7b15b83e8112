"""The C ABI on the CPU: every declared symbol is exported, and argument checks
fail with the documented status before anything is launched (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqm.h")

bqm = pytest.importorskip("bit_quantized_moe_amd._lib")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bqm.LIB_PATH):
        pytest.fail("libbqm.so is not built (python -m bit_quantized_moe_amd.build)")
    return bqm.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bqm_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bqm.EXPORTS)


def test_abi_version(lib):
    assert lib.bqm_abi_version() == 2


def _q(fmt=1, n=1, rows=4, cols=32, mode=0, codes=16, scales=16, sdec=16):
    return bqm.QTensorC(fmt, mode, n, rows, cols, codes, scales, sdec, 1, 0)


def test_quantize_rejects_bad_shapes_and_pointers(lib):
    q = _q(cols=24)
    st = lib.bqm_quantize_nvfp4(16, 1, None, C.byref(q), None, 0, None)
    assert st == -2 and "multiple of 16" in bqm.bqm_last_error()
    q = _q(codes=None)
    assert lib.bqm_quantize_nvfp4(16, 1, None, C.byref(q), None, 0, None) == -1
    q = _q(codes=17)
    assert lib.bqm_quantize_nvfp4(16, 1, None, C.byref(q), None, 0, None) == -3
    q = _q()
    assert lib.bqm_quantize_nvfp4(None, 1, None, C.byref(q), None, 0, None) == -1
    # per-tensor mode needs the amax workspace
    assert lib.bqm_quantize_nvfp4(16, 1, None, C.byref(q), None, 0, None) == -5
    q = _q(fmt=2, cols=64)
    assert lib.bqm_quantize_nvfp4(16, 1, None, C.byref(q), None, 0, None) == -1
    q = _q(fmt=2, cols=96)
    assert lib.bqm_quantize_nf4(16, C.byref(q), None) == -2
    q = _q(fmt=7)
    assert lib.bqm_dequantize(C.byref(q), 16, None) == -1
    q = _q(mode=5)
    assert lib.bqm_dequantize(C.byref(q), 16, None) == -1


def test_workspace_sizes(lib):
    assert lib.bqm_quantize_nvfp4_workspace_size(4, 64, 256, 1) == 0
    # the running amax of each matrix
    assert lib.bqm_quantize_nvfp4_workspace_size(4, 64, 256, 0) == 4 * 4
    assert lib.bqm_quantize_nvfp4_workspace_size(2, 4096, 6144, 0) == 2 * 4
    # per chunk of 2048 routed pairs: the E expert counts and the count of dropped pairs
    assert lib.bqm_permute_workspace_size(16384, 256, 8) == 64 * 257 * 4


def test_route_and_permute_reject_bad_args(lib):
    assert lib.bqm_route(16, 4, 8, 9, 0, 16, 16, None) == -2          # k > E
    assert lib.bqm_route(16, 4, 2000, 2, 0, 16, 16, None) == -2       # E too large
    assert lib.bqm_route(16, -1, 8, 2, 0, 16, 16, None) == -1
    assert lib.bqm_route(None, 4, 8, 2, 0, 16, 16, None) == -1
    assert lib.bqm_route(16, 4, 8, 2, 0, 20, 16, None) == -3
    assert lib.bqm_route(None, 0, 8, 2, 0, None, None, None) == 0     # T == 0 is a no-op
    assert lib.bqm_permute(16, 4, 8, 2, 16, 16, 16, None, 0, None) == -5
    assert lib.bqm_permute(16, 4, 8, 0, 16, 16, 16, 16, 4096, None) == -2
    assert lib.bqm_permute(16, 4, 8, 2, 16, 16, None, 16, 4096, None) == -1


def test_empty_inputs_are_noops(lib):
    q = _q(n=0)
    assert lib.bqm_quantize_nvfp4(None, 1, None, C.byref(q), None, 0, None) == 0
    assert lib.bqm_dequantize(C.byref(q), None, None) == 0
    q = _q(fmt=2, n=0, cols=64)
    assert lib.bqm_quantize_nf4(None, C.byref(q), None) == 0


def _desc(shared=0, T=64, H=256, I=128, E=8, k=2, r=8):
    gu = _q(n=E, rows=2 * I, cols=H)
    dn = _q(n=E, rows=H, cols=I)
    return bqm.MoEDescC(T, H, I, E, k, r, 0, 1.0, shared, gu, dn, 16, 16, 16, 16, None)


def test_moe_shared_lora_a_flag_and_workspace(lib):
    # host-side only: the descriptor check runs before any device work
    d = _desc(shared=3)
    assert lib.bqm_moe_fwd(C.byref(d), 16, 16, 16, 16, None, 0, None) == -1
    assert "lora_shared_a" in bqm.bqm_last_error()
    d = _desc(shared=1)
    assert lib.bqm_moe_fwd(C.byref(d), 16, 16, 16, 16, None, 0, None) == -5
    # the shared-A gradient adds its partial sums: min(E, 64) parts of the experts,
    # each [r, max(H, I)] FP32
    for T, E, split in ((64, 8, 8), (16384, 256, 64), (3000, 40, 40)):
        a = lib.bqm_moe_workspace_size(C.byref(_desc(0, T=T, E=E)))
        b = lib.bqm_moe_workspace_size(C.byref(_desc(1, T=T, E=E)))
        assert b - a == -(-split * 8 * 256 * 4 // 256) * 256, (T, E)


def test_nf4_nest_rejects_bad_arguments(lib):
    # host-side checks only (each call fails before any device work)
    def q(fmt=2, n=1, rows=4, cols=64, nested=0, sdec=16):
        return bqm.QTensorC(fmt, 0, n, rows, cols, 16, 16, sdec, 1, nested)
    plain, nested = q(), q(nested=1)
    bad = [(q(nested=1), nested, -1),            # plain side already nested
           (plain, q(nested=0), -1),             # target not marked nested
           (plain, q(nested=1, rows=8), -2),     # shapes differ
           (plain, q(nested=1, sdec=None), -1),  # nested needs the offset / group scales
           (plain, q(nested=2), -1),             # nested is 0 or 1
           (q(fmt=1, cols=64), nested, -1)]      # NVFP4 stacks cannot be nested
    for a, b, want in bad:
        assert lib.bqm_nf4_nest(C.byref(a), C.byref(b), None) == want, bqm.bqm_last_error()
    # the NF4 quantizer writes the plain form only; an NVFP4 stack cannot carry nested = 1
    assert lib.bqm_quantize_nf4(16, C.byref(q(nested=1)), None) == -1
    assert lib.bqm_quantize_nvfp4(16, 1, None, C.byref(q(fmt=1, cols=64, nested=1)), 16, 64, None) == -1
    # empty stacks are no-ops
    assert lib.bqm_nf4_nest(C.byref(q(n=0)), C.byref(q(n=0, nested=1)), None) == 0


def test_noalloc_quantizer_rejects_more_matrices_than_its_scratch(lib):
    # 65537 matrices would need 65537 running-amax slots: refused before any launch
    q = _q(n=65537, rows=1, cols=16)
    st = lib.bqm_quantize_nvfp4_noalloc(16, 1, None, C.byref(q), None)
    assert st == -5 and "65536" in bqm.bqm_last_error()
    q = _q(cols=24)
    assert lib.bqm_quantize_nvfp4_noalloc(16, 1, None, C.byref(q), None) == -2
