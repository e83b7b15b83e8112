"""ctypes binding of libbqm.so: one Python function per C entry point, same names.

Only argument marshalling happens here (tensor -> device pointer, sizes, stream
handle, status -> exception); every step of the path runs in the HIP library.
torch supplies device memory and streams.  The library must be built (python -m
bit_quantized_moe_amd.build); without it every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbqm.so")

FMT_NVFP4 = 1
FMT_NF4 = 2
SCALE_PER_TENSOR = 0
SCALE_PER_ROW = 1

STAGES = ["permute", "act_quant_x", "lora_a_gu", "gate_up_fwd", "act_quant_a", "lora_a_dn", "down_fwd",
          "combine_fwd", "dtopk", "lora_b_dn", "down_dgrad", "lora_b_gu", "gate_up_dgrad", "combine_dgrad",
          "lora_grad"]
STAGE_COUNT = len(STAGES)

STATUS = {0: "BQM_OK", -1: "BQM_ERR_INVALID_ARG", -2: "BQM_ERR_SHAPE", -3: "BQM_ERR_ALIGN",
          -4: "BQM_ERR_UNSUPPORTED", -5: "BQM_ERR_WORKSPACE", -6: "BQM_ERR_HIP"}

EXPORTS = ["bqm_abi_version", "bqm_last_error", "bqm_quantize_nvfp4_workspace_size",
           "bqm_quantize_nvfp4", "bqm_quantize_nvfp4_noalloc", "bqm_quantize_nf4", "bqm_dequantize", "bqm_route",
           "bqm_permute_workspace_size", "bqm_permute", "bqm_moe_workspace_size", "bqm_moe_fwd",
           "bqm_moe_dgrad", "bqm_moe_dgrad_colwise", "bqm_lora_grad", "bqm_nf4_nest"]


class BQMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class QTensorC(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("scale_mode", C.c_int32), ("n_mat", C.c_int64),
                ("rows", C.c_int64), ("cols", C.c_int64), ("codes", C.c_void_p),
                ("scales", C.c_void_p), ("s_dec", C.c_void_p), ("four_over_six", C.c_int32),
                ("nested", C.c_int32)]


class MoEDescC(C.Structure):
    _fields_ = [("T", C.c_int64), ("H", C.c_int64), ("I", C.c_int64), ("E", C.c_int32),
                ("k", C.c_int32), ("r", C.c_int32), ("act_quant", C.c_int32),
                ("lora_scale", C.c_float), ("lora_shared_a", C.c_int32), ("w_gu", QTensorC),
                ("w_dn", QTensorC), ("A_gu", C.c_void_p), ("B_gu", C.c_void_p),
                ("A_dn", C.c_void_p), ("B_dn", C.c_void_p), ("stage_events", C.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libbqm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m bit_quantized_moe_amd.build")
    # torch first, so that the library binds to the HIP runtime torch already uses
    # (same soname: one runtime per process, shared streams and allocations)
    import torch  # noqa: F401
    lib = C.CDLL(path)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "bqm_abi_version": (C.c_int, []),
        "bqm_last_error": (C.c_char_p, []),
        "bqm_quantize_nvfp4_workspace_size": (sz, [i64, i64, i64, i32]),
        "bqm_quantize_nvfp4": (C.c_int, [vp, i32, vp, C.POINTER(QTensorC), vp, sz, vp]),
        "bqm_quantize_nvfp4_noalloc": (C.c_int, [vp, i32, vp, C.POINTER(QTensorC), vp]),
        "bqm_quantize_nf4": (C.c_int, [vp, C.POINTER(QTensorC), vp]),
        "bqm_nf4_nest": (C.c_int, [C.POINTER(QTensorC), C.POINTER(QTensorC), vp]),
        "bqm_dequantize": (C.c_int, [C.POINTER(QTensorC), vp, vp]),
        "bqm_route": (C.c_int, [vp, i64, i32, i32, i32, vp, vp, vp]),
        "bqm_permute_workspace_size": (sz, [i64, i32, i32]),
        "bqm_permute": (C.c_int, [vp, i64, i32, i32, vp, vp, vp, vp, sz, vp]),
        "bqm_moe_workspace_size": (sz, [C.POINTER(MoEDescC)]),
        "bqm_moe_fwd": (C.c_int, [C.POINTER(MoEDescC), vp, vp, vp, vp, vp, sz, vp]),
        "bqm_moe_dgrad": (C.c_int, [C.POINTER(MoEDescC), vp, vp, sz, vp, vp, vp]),
        "bqm_moe_dgrad_colwise": (C.c_int, [C.POINTER(MoEDescC), C.POINTER(QTensorC), C.POINTER(QTensorC), vp, vp,
                                            sz, vp, vp, vp]),
        "bqm_lora_grad": (C.c_int, [C.POINTER(MoEDescC), vp, vp, vp, sz, vp, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = _lib.bqm_last_error().decode(errors="replace")
        raise BQMError(status, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


@dataclass
class QTensor:
    """A rowwise-quantized stack held in torch tensors (see bqm_qtensor)."""
    fmt: int
    scale_mode: int
    n_mat: int
    rows: int
    cols: int
    codes: object
    scales: object
    s_dec: object = None
    four_over_six: int = 1
    nested: int = 0          # NF4: 1 = double-quantized absmax (see bqm_nf4_nest)

    def c(self) -> QTensorC:
        return QTensorC(self.fmt, self.scale_mode, self.n_mat, self.rows, self.cols, _ptr(self.codes),
                        _ptr(self.scales), _ptr(self.s_dec), self.four_over_six, int(self.nested))


def nf4_nest_groups(rows, cols) -> int:
    """Groups of 256 absmax blocks per matrix of a nested NF4 stack."""
    return -(-(rows * cols // 64) // 256)


def alloc_qtensor(fmt, n_mat, rows, cols, device="cuda", scale_mode=SCALE_PER_TENSOR,
                  four_over_six=1, nested=0) -> QTensor:
    import torch
    codes = torch.empty((n_mat, rows, cols // 2), dtype=torch.uint8, device=device)
    if fmt == FMT_NVFP4:
        scales = torch.empty((n_mat, rows, cols // 16), dtype=torch.uint8, device=device)
        n = n_mat if scale_mode == SCALE_PER_TENSOR else n_mat * rows
        s_dec = torch.empty((max(n, 1),), dtype=torch.float32, device=device)
    elif nested:
        scales = torch.empty((n_mat, rows, cols // 64), dtype=torch.uint8, device=device)
        s_dec = torch.empty((max(n_mat, 1), 1 + nf4_nest_groups(rows, cols)), dtype=torch.float32, device=device)
    else:
        scales = torch.empty((n_mat, rows, cols // 64), dtype=torch.float32, device=device)
        s_dec = None
    return QTensor(fmt, scale_mode, n_mat, rows, cols, codes, scales, s_dec, four_over_six, nested)


def quantize_stack(w, fmt: str, stream=None) -> QTensor:
    """Allocate and fill a rowwise-quantized stack from a bf16 [n_mat, rows, cols] tensor:
    fmt "nvfp4" (per-tensor scale, Four-Over-Six), "nf4" or "nf4_nested" (NF4, then
    bqm_nf4_nest; the nested stack keeps the plain codes).  Allocation plus the library
    calls, nothing else."""
    import torch
    n_mat, rows, cols = w.shape
    if fmt == "nvfp4":
        q = alloc_qtensor(FMT_NVFP4, n_mat, rows, cols, device=w.device)
        wsb = bqm_quantize_nvfp4_workspace_size(n_mat, rows, cols, SCALE_PER_TENSOR)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=w.device)
        bqm_quantize_nvfp4(w, 1, None, q, ws, stream)
        return q
    if fmt not in ("nf4", "nf4_nested"):
        raise ValueError(f"unknown weight format {fmt!r}")
    q = alloc_qtensor(FMT_NF4, n_mat, rows, cols, device=w.device)
    bqm_quantize_nf4(w, q, stream)
    if fmt == "nf4":
        return q
    n = alloc_qtensor(FMT_NF4, n_mat, rows, cols, device=w.device, nested=1)
    n.codes = q.codes
    bqm_nf4_nest(q, n, stream)
    torch.cuda.synchronize()        # the plain FP32 absmax (q.scales) is freed on return
    return n


# ----------------------------------------------------------------------------
# one wrapper per entry point
# ----------------------------------------------------------------------------
def bqm_abi_version() -> int:
    return load().bqm_abi_version()


def bqm_last_error() -> str:
    return load().bqm_last_error().decode(errors="replace")


def bqm_quantize_nvfp4_workspace_size(n_mat, rows, cols, scale_mode) -> int:
    return load().bqm_quantize_nvfp4_workspace_size(n_mat, rows, cols, scale_mode)


def bqm_quantize_nvfp4(x, four_over_six: int, s_dec_in, out: QTensor, ws=None, stream=None):
    lib = load()
    qc = out.c()
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.bqm_quantize_nvfp4(_ptr(x), int(four_over_six), _ptr(s_dec_in), C.byref(qc), _ptr(ws),
                                  wsb, _stream(stream)))
    out.four_over_six = qc.four_over_six
    return out


def bqm_quantize_nvfp4_noalloc(x, four_over_six: int, s_dec_in, out: QTensor, stream=None):
    lib = load()
    qc = out.c()
    _check(lib.bqm_quantize_nvfp4_noalloc(_ptr(x), int(four_over_six), _ptr(s_dec_in), C.byref(qc),
                                          _stream(stream)))
    out.four_over_six = qc.four_over_six
    return out


def bqm_quantize_nf4(x, out: QTensor, stream=None):
    lib = load()
    qc = out.c()
    _check(lib.bqm_quantize_nf4(_ptr(x), C.byref(qc), _stream(stream)))
    return out


def bqm_nf4_nest(plain: QTensor, nested: QTensor, stream=None):
    lib = load()
    pc, nc = plain.c(), nested.c()
    _check(lib.bqm_nf4_nest(C.byref(pc), C.byref(nc), _stream(stream)))
    return nested


def bqm_dequantize(q: QTensor, y, stream=None):
    lib = load()
    qc = q.c()
    _check(lib.bqm_dequantize(C.byref(qc), _ptr(y), _stream(stream)))
    return y


def bqm_route(logits, T, E, k, renorm, topk_idx, topk_w, stream=None):
    _check(load().bqm_route(_ptr(logits), T, E, k, int(renorm), _ptr(topk_idx), _ptr(topk_w),
                            _stream(stream)))


def bqm_permute_workspace_size(T, E, k) -> int:
    return load().bqm_permute_workspace_size(T, E, k)


def bqm_permute(topk_idx, T, E, k, perm, inv, offsets, ws, stream=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().bqm_permute(_ptr(topk_idx), T, E, k, _ptr(perm), _ptr(inv), _ptr(offsets),
                              _ptr(ws), wsb, _stream(stream)))


@dataclass
class MoEDesc:
    T: int
    H: int
    I: int
    E: int
    k: int
    r: int
    w_gu: QTensor
    w_dn: QTensor
    A_gu: object = None
    B_gu: object = None
    A_dn: object = None
    B_dn: object = None
    lora_scale: float = 1.0
    act_quant: int = 0
    stage_events: Optional[int] = None   # address of a host array of 2*STAGE_COUNT hipEvent_t
    lora_shared_a: int = 0               # 1: A_gu [r, H] and A_dn [r, I] shared by all experts

    def c(self) -> MoEDescC:
        return MoEDescC(self.T, self.H, self.I, self.E, self.k, self.r, int(self.act_quant),
                        float(self.lora_scale), int(self.lora_shared_a), self.w_gu.c(), self.w_dn.c(), _ptr(self.A_gu),
                        _ptr(self.B_gu), _ptr(self.A_dn), _ptr(self.B_dn), self.stage_events)


def bqm_moe_workspace_size(d: MoEDesc) -> int:
    dc = d.c()
    return load().bqm_moe_workspace_size(C.byref(dc))


def bqm_moe_fwd(d: MoEDesc, x, topk_idx, topk_w, out, ws, stream=None):
    dc = d.c()
    _check(load().bqm_moe_fwd(C.byref(dc), _ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(out), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)))


def bqm_moe_dgrad(d: MoEDesc, dy, ws, dx, dtopk_w=None, stream=None):
    dc = d.c()
    _check(load().bqm_moe_dgrad(C.byref(dc), _ptr(dy), _ptr(ws), ws.numel() * ws.element_size(),
                                _ptr(dx), _ptr(dtopk_w), _stream(stream)))


def bqm_moe_dgrad_colwise(d: MoEDesc, w_gu_col: QTensor, w_dn_col: QTensor, dy, ws, dx, dtopk_w=None, stream=None):
    dc = d.c()
    gc, nc = w_gu_col.c(), w_dn_col.c()
    _check(load().bqm_moe_dgrad_colwise(C.byref(dc), C.byref(gc), C.byref(nc), _ptr(dy), _ptr(ws),
                                        ws.numel() * ws.element_size(), _ptr(dx), _ptr(dtopk_w), _stream(stream)))


def bqm_lora_grad(d: MoEDesc, x, dy, ws, dA_gu, dB_gu, dA_dn, dB_dn, stream=None):
    dc = d.c()
    _check(load().bqm_lora_grad(C.byref(dc), _ptr(x), _ptr(dy), _ptr(ws), ws.numel() * ws.element_size(),
                                _ptr(dA_gu), _ptr(dB_gu), _ptr(dA_dn), _ptr(dB_dn), _stream(stream)))
