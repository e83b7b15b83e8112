"""Routed-expert MoE layer over 4-bit expert weights with a bf16 LoRA, in float64.

Test infrastructure (see the package docstring).

The layer is a plain definition, so this module writes the definition out in
float64 over the exactly dequantized weights W~ = DQ(Q(W)):

forward ("nf4moe - QLoRA for a 743B Fused-MoE", the QuantizedNaiveMoe forward;
the gate/up halves come from chunk(2, -1) of the gate_up product, the result is
act(gate) * up, and index_add_ adds each expert output times its routing weight
back onto its token):
    h   = X~ W~_gu^T + s (X A_gu^T) B_gu^T          X~ = X, or DQ(Q_row(X)) in W4A4
    g,u = h[:, :I], h[:, I:]
    a   = silu(g) * u,  a_b = bf16(a)               rounding point R1
    y   = a~ W~_dn^T + s (a_b A_dn^T) B_dn^T        a~ = a_b, or DQ(Q_row(a_b)) in W4A4
    out[t] = sum_j w[t, j] y[(t, j)]

dgrad, the input gradient through the same dequantized weights ("Getting
GLM-5.2 NVFP4 Post-Training off the ground", section "The 4-bit base that was
actually using 8-bit memory": the rowwise copy is dequantized to bf16 and the
backward contracts over the output dimension, dX = dY W; "The 4-bitter Lesson",
section "Improving Gradient Stability": the backward consumes DQ(Q(w))):
    da_u  = dOut[t] W~_dn + s (dOut[t] B_dn) A_dn
    dw[t,j] = <dOut[t], y[(t,j)]>
    da    = w da_u;  dg = da u sig(g)(1 + g(1 - sig(g)));  du = da silu(g)
    dh_b  = bf16([dg, du])                          rounding point R2
    dX[t] = sum_j ( dh_b W~_gu + s (dh_b B_gu) A_gu )

LoRA weight gradients (the adapter is the only trained part; per-expert A and B
on the 3-D stacks, "nf4moe", section "Does it actually train?"):
    dB_gu = s dh_b^T (X A_gu^T)        dA_gu = s (dh_b B_gu)^T X
    dB_dn = s (w dOut)^T (a_b A_dn^T)  dA_dn = s (w dOut B_dn)^T a_b
Experts that receive no token get exact zeros.

Shared-A layout ("Getting GLM-5.2 NVFP4 Post-Training off the ground", its
serving part, the paragraph on the non-fused NVFP4 MoE-LoRA path: the adapter
there has one LoRA-A common to all experts and a LoRA-B per expert): A_gu
is [r, H] and A_dn [r, I], used by every expert in the formulas above, and
dA_gu, dA_dn are the sums of those per-expert terms over all experts (the
gradient of one matrix that every expert reads).

Readings: s (the LoRA scale) defaults to 1, the pages give no alpha; LoRA reads
the unquantized bf16 activations in W4A4; the activation quantizers are the
identity in the backward (straight-through), the backward keeping bf16
operands.  R1 and R2 are the only roundings: they are the bf16 operands the
path defines.  round_points=False gives the pure float64 chain.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import formats as fm
from . import quant as oq


@dataclass
class MoEWeights:
    fmt: str                    # "nvfp4" or "nf4"
    gu: object                  # NVFP4Tensor / NF4Tensor over [E, 2I, H]
    dn: object                  # NVFP4Tensor / NF4Tensor over [E, H, I]
    A_gu: Optional[np.ndarray]  # [E, r, H]  (bf16 values); [r, H] when shared_a
    B_gu: Optional[np.ndarray]  # [E, 2I, r]
    A_dn: Optional[np.ndarray]  # [E, r, I]; [r, I] when shared_a
    B_dn: Optional[np.ndarray]  # [E, H, r]
    lora_scale: float = 1.0
    act_quant: bool = False     # W4A4: per-token NVFP4 (+4/6) activations in the base GEMMs
    shared_a: bool = False      # one LoRA-A for all experts, per-expert LoRA-B

    @property
    def r(self) -> int:
        return 0 if self.A_gu is None else self.A_gu.shape[-2]

    def a_gu(self, e: int) -> np.ndarray:
        return (self.A_gu if self.shared_a else self.A_gu[e]).astype(np.float64)

    def a_dn(self, e: int) -> np.ndarray:
        return (self.A_dn if self.shared_a else self.A_dn[e]).astype(np.float64)


class LazyExperts:
    """An expert stack quantized by this oracle one expert at a time, on first use.

    fetch(e) returns expert e's bf16 weights as float32 [rows, cols]; fmt is
    "nvfp4" (per-tensor scale, Four-Over-Six), "nf4" or "nf4_nested" (NF4 with the
    double-quantized absmax, nested per expert matrix).  Used for the full-size
    workloads, where only the experts a sampled token touches are needed.
    """

    def __init__(self, fetch, fmt: str, four_over_six: bool = True):
        self.fetch, self.fmt, self.fos = fetch, fmt, four_over_six
        self.cache = {}

    def matrix(self, e: int) -> np.ndarray:
        if e not in self.cache:
            x = fm.f32(self.fetch(e))[None]
            if self.fmt == "nvfp4":
                self.cache[e] = oq.dequantize_nvfp4_exact(oq.quantize_nvfp4(x, self.fos))[0]
            elif self.fmt == "nf4_nested":
                self.cache[e] = oq.dequantize_nf4_nested(oq.nest_absmax(oq.quantize_nf4(x)))[0].astype(np.float64)
            else:
                self.cache[e] = oq.dequantize_nf4(oq.quantize_nf4(x))[0].astype(np.float64)
        return self.cache[e]


class ColumnwiseExperts:
    """The second, columnwise quantization of an expert stack that FP4 tensor cores need
    for the dgrad (GLM page, section "Why can't we just transpose the one copy?"): each
    expert's W_e^T is quantized rowwise (NVFP4, per-tensor scale, Four-Over-Six), i.e.
    with its 16-blocks along W_e's rows, and matrix(e) returns DQ(Q(W_e^T))^T, which
    stands where the rowwise DQ(Q(W_e)) stands in the dgrad.  fetch(e) returns W_e as
    float32 [rows, cols]."""

    def __init__(self, fetch, four_over_six: bool = True):
        self.fetch, self.fos = fetch, four_over_six
        self.cache = {}

    def matrix(self, e: int) -> np.ndarray:
        if e not in self.cache:
            xt = np.ascontiguousarray(fm.f32(self.fetch(e)).T)[None]
            self.cache[e] = oq.dequantize_nvfp4_exact(oq.quantize_nvfp4(xt, self.fos))[0].T
        return self.cache[e]


def expert_matrix(q, e: int) -> np.ndarray:
    """Exact float64 DQ of expert e's 2-D slice (the GEMM operand)."""
    if isinstance(q, (LazyExperts, ColumnwiseExperts)):
        return q.matrix(e)
    if isinstance(q, oq.NVFP4Tensor):
        one = oq.NVFP4Tensor(q.codes[e:e + 1], q.scales[e:e + 1], q.s_dec[e:e + 1],
                             q.four_over_six, q.per_row)
        return oq.dequantize_nvfp4_exact(one)[0]
    if isinstance(q, oq.NF4Nested):
        one = oq.NF4Nested(q.codes[e:e + 1], q.absmax_q[e:e + 1], q.group_scale[e:e + 1], q.offset[e:e + 1])
        return oq.dequantize_nf4_nested(one)[0].astype(np.float64)
    one = oq.NF4Tensor(q.codes[e:e + 1], q.absmax[e:e + 1])
    return oq.dequantize_nf4(one)[0].astype(np.float64)


def act_dq(rows_bf16: np.ndarray) -> np.ndarray:
    """DQ(Q_row(rows)) exactly, per-token NVFP4 with Four-Over-Six (W4A4 operand)."""
    q = oq.quantize_nvfp4(fm.f32(rows_bf16)[None], four_over_six=True, per_row=True)
    return oq.dequantize_nvfp4_exact(q)[0]


def silu(g):
    return g / (1.0 + np.exp(-g))


def sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def _bf16(a: np.ndarray) -> np.ndarray:
    return fm.bf16_round(a.astype(np.float32)).astype(np.float64)


def _pairs_by_expert(topk_idx, tokens):
    """Routed pairs f = t*k + j of the selected tokens, grouped by expert, f ascending."""
    ti = np.asarray(topk_idx, dtype=np.int64)
    T, k = ti.shape
    toks = np.arange(T) if tokens is None else np.sort(np.asarray(tokens, dtype=np.int64))
    f = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    ex = ti.reshape(-1)[f]
    order = np.lexsort((f, ex))
    f, ex = f[order], ex[order]
    groups = {}
    for e in np.unique(ex):
        groups[int(e)] = f[ex == e]
    return groups, k


def forward(w: MoEWeights, x, topk_idx, topk_w, tokens=None, round_points: bool = True,
            experts=None):
    """Forward pass.  Returns (out rows [len(tokens) or T, H], cache for dgrad).

    tokens: optional subset of token ids (their rows of out are exact, since
    every expert touches a token only through that token's own routed rows).
    experts: optional subset of experts to evaluate (then out is partial).
    """
    x64 = np.asarray(x, dtype=np.float64)
    T, H = x64.shape
    tw = np.asarray(topk_w, dtype=np.float64)
    groups, k = _pairs_by_expert(topk_idx, tokens)
    s = float(w.lora_scale)
    r = w.r
    cache = {"groups": groups, "k": k, "per_expert": {}}
    y_rows = {}
    for e, fs in groups.items():
        if experts is not None and e not in experts:
            continue
        t = fs // k
        X = x64[t]
        Xt = act_dq(X) if w.act_quant else X
        Wgu = expert_matrix(w.gu, e)
        h = Xt @ Wgu.T
        U_gu = X @ w.a_gu(e).T if r else None
        if r:
            h = h + s * (U_gu @ w.B_gu[e].astype(np.float64).T)
        I = h.shape[1] // 2
        g, u = h[:, :I], h[:, I:]
        a = silu(g) * u
        a_b = _bf16(a) if round_points else a
        at = act_dq(a_b) if w.act_quant else a_b
        Wdn = expert_matrix(w.dn, e)
        y = at @ Wdn.T
        U_dn = a_b @ w.a_dn(e).T if r else None
        if r:
            y = y + s * (U_dn @ w.B_dn[e].astype(np.float64).T)
        cache["per_expert"][e] = dict(fs=fs, t=t, X=X, g=g, u=u, a_b=a_b, y=y,
                                      U_gu=U_gu, U_dn=U_dn, Wgu=None, Wdn=None)
        for i, f in enumerate(fs):
            y_rows[int(f)] = y[i]
    toks = np.arange(T) if tokens is None else np.sort(np.asarray(tokens, dtype=np.int64))
    out = np.zeros((toks.size, H))
    for n, t in enumerate(toks):
        acc = np.zeros(H)
        for j in range(k):
            f = int(t) * k + j
            if f in y_rows:
                acc = acc + tw[t, j] * y_rows[f]
        out[n] = acc
    cache["tokens"] = toks
    cache["y_rows"] = y_rows
    return out, cache


def dgrad(w: MoEWeights, cache, dout, topk_w, round_points: bool = True):
    """Input gradient and routing-weight gradient; also returns what the LoRA grads need.

    dout: [T, H] (rows of the cached tokens are read).  Returns (dX rows for
    cache["tokens"], dtopk_w [T, k] (zeros outside the cached tokens), bwd cache).
    """
    d64 = np.asarray(dout, dtype=np.float64)
    tw = np.asarray(topk_w, dtype=np.float64)
    k = cache["k"]
    s = float(w.lora_scale)
    r = w.r
    T = tw.shape[0]
    H = d64.shape[1]
    dtw = np.zeros((T, k))
    dx_rows = {}
    bwd = {}
    for e, c in cache["per_expert"].items():
        fs, t = c["fs"], c["t"]
        j = fs % k
        dO = d64[t]
        Wdn = expert_matrix(w.dn, e)
        da_u = dO @ Wdn
        V_dn = dO @ w.B_dn[e].astype(np.float64) if r else None
        if r:
            da_u = da_u + s * (V_dn @ w.a_dn(e))
        dtw[t, j] = np.einsum("nh,nh->n", dO, c["y"])
        wr = tw[t, j][:, None]
        da = wr * da_u
        g, u = c["g"], c["u"]
        sg = sigmoid(g)
        dg = da * u * sg * (1.0 + g * (1.0 - sg))
        du = da * (g * sg)
        dh = np.concatenate([dg, du], axis=1)
        dh_b = _bf16(dh) if round_points else dh
        Wgu = expert_matrix(w.gu, e)
        dxr = dh_b @ Wgu
        V_gu = dh_b @ w.B_gu[e].astype(np.float64) if r else None
        if r:
            dxr = dxr + s * (V_gu @ w.a_gu(e))
        for i, f in enumerate(fs):
            dx_rows[int(f)] = dxr[i]
        bwd[e] = dict(dh_b=dh_b, V_gu=V_gu, V_dn=V_dn, wr=wr, dO=dO)
    toks = cache["tokens"]
    dX = np.zeros((toks.size, H))
    for n, t in enumerate(toks):
        acc = np.zeros(H)
        for jj in range(k):
            f = int(t) * k + jj
            if f in dx_rows:
                acc = acc + dx_rows[f]
        dX[n] = acc
    return dX, dtw, bwd


def lora_grad(w: MoEWeights, cache, bwd, E: int):
    """LoRA gradients (float64): dA_gu [E,r,H], dB_gu [E,2I,r], dA_dn [E,r,I], dB_dn [E,H,r];
    with shared_a, dA_gu [r,H] and dA_dn [r,I] are the sums over the experts."""
    r = w.r
    s = float(w.lora_scale)
    H = w.A_gu.shape[-1]
    I = w.A_dn.shape[-1]
    dA_gu = np.zeros((E, r, H))
    dB_gu = np.zeros((E, 2 * I, r))
    dA_dn = np.zeros((E, r, I))
    dB_dn = np.zeros((E, H, r))
    for e, c in cache["per_expert"].items():
        b = bwd[e]
        dB_gu[e] = s * (b["dh_b"].T @ c["U_gu"])
        dA_gu[e] = s * (b["V_gu"].T @ c["X"])
        wdO = b["wr"] * b["dO"]
        dB_dn[e] = s * (wdO.T @ c["U_dn"])
        dA_dn[e] = s * ((b["wr"] * b["V_dn"]).T @ c["a_b"])
    if w.shared_a:
        return dA_gu.sum(axis=0), dB_gu, dA_dn.sum(axis=0), dB_dn
    return dA_gu, dB_gu, dA_dn, dB_dn


def rel_errors(got, ref):
    """(||G-R||_F / ||R||_F, max|G-R| / max|R|): the two parity measures for float outputs."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    nr = np.linalg.norm(r)
    mr = np.abs(r).max() if r.size else 0.0
    d = g - r
    fro = np.linalg.norm(d) / nr if nr > 0 else np.linalg.norm(d)
    mx = np.abs(d).max() / mr if mr > 0 else (np.abs(d).max() if d.size else 0.0)
    return float(fro), float(mx)
