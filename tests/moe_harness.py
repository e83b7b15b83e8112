"""Runs the MoE layer through the C ABI and through the oracle on the same seeded inputs.

The GPU side quantizes the bf16 weights with the library, routes the logits
with the library and runs forward, dgrad and LoRA gradients.  The oracle side
quantizes the same bf16 weights itself (only the experts it needs), routes the
same logits itself and evaluates the float64 definition.  Nothing flows from
the GPU results into the oracle.
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import moe as om
from oracle import routing as orr


def _bqm():
    import bit_quantized_moe_amd as bqm
    return bqm


def quantize_stack_gpu(w, fmt):
    return _bqm().quantize_stack(w, fmt)


def poison_experts(q, experts, fmt):
    """Make the scales of the given experts decode to NaN (E4M3 0x7F / NaN absmax)."""
    import torch
    for e in experts:
        if fmt in ("nvfp4", "nf4_nested"):
            q.scales[e].fill_(0x7F)
        else:
            q.scales[e].fill_(float("nan"))
    torch.cuda.synchronize()


def colwise_stacks_gpu(inp: synth.LayerInputs, dev):
    """The columnwise copies Q(W_gu^T) [E, H, 2I] and Q(W_dn^T) [E, I, H] (NVFP4, per-tensor)."""
    wgu_t = inp.w_gu.to(dev).transpose(1, 2).contiguous()
    wdn_t = inp.w_dn.to(dev).transpose(1, 2).contiguous()
    return quantize_stack_gpu(wgu_t, "nvfp4"), quantize_stack_gpu(wdn_t, "nvfp4")


def gpu_layer(inp: synth.LayerInputs, dev, lora_scale=1.0, poison_empty=False, lora=True, colwise=False):
    """Forward + dgrad (+ LoRA grads) on the GPU.  Returns a dict of torch tensors.
    colwise: the dgrad runs over columnwise copies of the weights (bqm_moe_dgrad_colwise)."""
    import torch
    bqm = _bqm()
    s = inp.shape
    x = inp.x.to(dev)
    lg = inp.logits.to(dev)
    dout = inp.dout.to(dev)
    qgu = quantize_stack_gpu(inp.w_gu.to(dev), s.fmt)
    qdn = quantize_stack_gpu(inp.w_dn.to(dev), s.fmt)
    idx = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
    tw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    if s.T:
        bqm.bqm_route(lg, s.T, s.E, s.k, 0, idx, tw)
    if poison_empty:
        hit = torch.zeros(s.E, dtype=torch.bool, device=dev)
        hit[idx.long().reshape(-1)] = True
        empty = torch.nonzero(~hit).reshape(-1).tolist()
        poison_experts(qgu, empty, s.fmt)
        poison_experts(qdn, empty, s.fmt)
    lor = {}
    if s.r:
        lor = dict(A_gu=inp.A_gu.to(dev), B_gu=inp.B_gu.to(dev), A_dn=inp.A_dn.to(dev), B_dn=inp.B_dn.to(dev))
    d = bqm.MoEDesc(s.T, s.H, s.I, s.E, s.k, s.r, qgu, qdn, lora_scale=lora_scale,
                    act_quant=int(s.act_quant), lora_shared_a=int(s.shared_a), **lor)
    ws = torch.empty(max(bqm.bqm_moe_workspace_size(d), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev)
    bqm.bqm_moe_fwd(d, x, idx, tw, out, ws)
    dx = torch.empty_like(out)
    dtw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    if colwise:
        cgu, cdn = colwise_stacks_gpu(inp, dev)
        bqm.bqm_moe_dgrad_colwise(d, cgu, cdn, dout, ws, dx, dtw)
    else:
        bqm.bqm_moe_dgrad(d, dout, ws, dx, dtw)
    res = dict(idx=idx, tw=tw, out=out, dx=dx, dtw=dtw, desc=d, ws=ws)
    if s.r and lora:
        ea = () if s.shared_a else (s.E,)
        g = dict(dA_gu=torch.empty(ea + (s.r, s.H), dtype=torch.float32, device=dev),
                 dB_gu=torch.empty((s.E, 2 * s.I, s.r), dtype=torch.float32, device=dev),
                 dA_dn=torch.empty(ea + (s.r, s.I), dtype=torch.float32, device=dev),
                 dB_dn=torch.empty((s.E, s.H, s.r), dtype=torch.float32, device=dev))
        bqm.bqm_lora_grad(d, x, dout, ws, g["dA_gu"], g["dB_gu"], g["dA_dn"], g["dB_dn"])
        res.update(g)
    torch.cuda.synchronize()
    return res


class HostInputs:
    """Host (float32 numpy) views of the layer inputs the oracle reads; weights per expert on demand."""

    def __init__(self, inp: synth.LayerInputs):
        self.shape = inp.shape
        self.x = synth.f32_numpy(inp.x)
        self.dout = synth.f32_numpy(inp.dout)
        self.logits = inp.logits.float().cpu().numpy()
        s = inp.shape
        self.lora = None
        if s.r:
            self.lora = [synth.f32_numpy(t) for t in (inp.A_gu, inp.B_gu, inp.A_dn, inp.B_dn)]
        self._wgu, self._wdn = inp.w_gu, inp.w_dn

    def weights(self, lora_scale=1.0):
        s = self.shape
        gu = om.LazyExperts(lambda e: synth.f32_numpy(self._wgu[e]), s.fmt)
        dn = om.LazyExperts(lambda e: synth.f32_numpy(self._wdn[e]), s.fmt)
        lo = self.lora if self.lora is not None else [None] * 4
        return om.MoEWeights(s.fmt, gu, dn, *lo, lora_scale=lora_scale, act_quant=s.act_quant,
                             shared_a=s.shared_a)

    def weights_colwise(self, lora_scale=1.0):
        """The same layer with the oracle's columnwise copies (DQ(Q(W^T))^T) as base weights."""
        s = self.shape
        gu = om.ColumnwiseExperts(lambda e: synth.f32_numpy(self._wgu[e]))
        dn = om.ColumnwiseExperts(lambda e: synth.f32_numpy(self._wdn[e]))
        lo = self.lora if self.lora is not None else [None] * 4
        return om.MoEWeights("nvfp4", gu, dn, *lo, lora_scale=lora_scale, act_quant=s.act_quant,
                             shared_a=s.shared_a)


def _bf16_neighbours(a):
    """For float64 values: (nearest bf16, the other bf16 neighbour, distance to the rounding midpoint)."""
    from oracle import formats as fm
    a32 = a.astype(np.float32)
    near = fm.bf16_round(a32).astype(np.float64)
    bits = a32.view(np.uint32) & np.uint32(0xFFFF0000)
    lo = bits.view(np.float32).astype(np.float64)                      # truncation toward zero
    hi = (bits + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    other = np.where(near == lo, hi, lo)
    mid = (lo + hi) / 2
    return near, other, np.abs(a - mid)


U32 = 2.0 ** -24          # FP32 unit roundoff
H_ERR_FACTOR = 2.0        # |h_gpu - h| <= H_ERR_FACTOR * U32 * sum_k |p_k| (see below)


def w4a4_a_error_bound(c, w, e):
    """Per-element bound on how far the GPU's FP32 a = silu(g) * u can lie from the
    oracle's float64 a, for expert e's rows (cache entry c).

    The GPU forms g and u as FP32 sums of exact bf16 x bf16 products p_k (the MFMA
    accumulates in FP32): the first-order bound of such a sum is gamma_n * sum|p_k|
    with gamma_n ~ n u for n sequential roundings; measured on the GPU over 3.5M
    elements of two W4A4 layers, |h_gpu - h| stays below 1.1 u sum|p_k| (the rounding
    errors of the K/16 accumulation steps largely cancel), so the bound taken is
    2 u sum|p_k| over the base and LoRA products, plus 2 u |h| for the per-row and
    per-expert scale multiplications.  It propagates to a through
    da = silu'(g) u dg + silu(g) du, plus 4 u |a| for the FP32 evaluation of silu * u."""
    X = om.act_dq(c["X"])
    Wg = om.expert_matrix(w.gu, e)
    S = np.abs(X) @ np.abs(Wg).T
    if w.r:
        S = S + abs(w.lora_scale) * (np.abs(c["U_gu"]) @ np.abs(w.B_gu[e].astype(np.float64)).T)
    g, u = c["g"], c["u"]
    I = g.shape[1]
    Bh = H_ERR_FACTOR * U32 * S + 2 * U32 * np.abs(np.concatenate([g, u], axis=1))
    sg = om.sigmoid(g)
    dsilu = sg * (1.0 + g * (1.0 - sg))
    a = om.silu(g) * u
    return np.abs(dsilu * u) * Bh[:, :I] + np.abs(om.silu(g)) * Bh[:, I:] + 4 * U32 * np.abs(a)


def resolve_w4a4_alternatives(g_out, g_dtw, o, h: HostInputs):
    """W4A4 quantizes a = silu(g) u per token after a GEMM.  Where an element of a
    lies closer to a bf16 rounding midpoint than the FP32 error bound of the GPU's
    a (w4a4_a_error_bound), either rounding is a valid result of FP32 accumulation,
    and when that element decides the row's amax the whole row is quantized with
    the neighbouring scale.  For every such routed row this evaluates the
    alternative with the oracle's own arithmetic and keeps, per token, the valid
    combination closest to the GPU result (out and dtopk_w rows of the oracle
    result are replaced).  Returns the number of rows that had an alternative."""
    s = h.shape
    if not s.act_quant:
        return 0
    w = o["w"]
    k = s.k
    tokens = list(o["tokens"])
    row_of = {int(t): n for n, t in enumerate(tokens)}
    cache = o["cache"]
    n_alt = 0
    for e, c in cache["per_expert"].items():
        a = om.silu(c["g"]) * c["u"]
        near, other, dist = _bf16_neighbours(a)
        amb = dist <= w4a4_a_error_bound(c, w, e)
        amax = np.abs(near).max(axis=1)
        Wdn = om.expert_matrix(w.dn, e)
        for i in range(a.shape[0]):
            cand = np.nonzero(amb[i] & ((np.abs(other[i]) > amax[i]) | (np.abs(near[i]) == amax[i])))[0]
            if cand.size == 0:
                continue
            f = int(c["fs"][i])
            t, j = f // k, f % k
            if t not in row_of:
                continue
            n = row_of[t]
            wt = o["tw"][t, j]
            best = None
            for col in cand:
                alt = near[i].copy()
                alt[col] = other[i][col]
                y_alt = om.act_dq(alt[None])[0] @ Wdn.T
                if w.r:
                    y_alt = y_alt + w.lora_scale * ((alt @ w.a_dn(e).T)
                                                    @ w.B_dn[e].astype(np.float64).T)
                out_alt = o["out"][n] - wt * c["y"][i] + wt * y_alt
                err = np.abs(out_alt - g_out[n]).max()
                if best is None or err < best[0]:
                    best = (err, out_alt, float(h.dout[t].astype(np.float64) @ y_alt))
            err0 = np.abs(o["out"][n] - g_out[n]).max()
            if best[0] < err0:
                o["out"][n] = best[1]
                o["dtw"][t, j] = best[2]
            n_alt += 1
    return n_alt


def oracle_layer(h: HostInputs, lora_scale=1.0, tokens=None, lora_experts=None, colwise=False):
    """Oracle forward + dgrad for the chosen tokens (all if None), and LoRA grads
    for lora_experts (all experts if None and tokens is None).  colwise: the dgrad
    uses the columnwise copies DQ(Q(W^T))^T."""
    s = h.shape
    w = h.weights(lora_scale)
    wd = h.weights_colwise(lora_scale) if colwise else w
    idx, tw = orr.route(h.logits, s.k)
    out, cache = om.forward(w, h.x, idx, tw, tokens=tokens)
    dx, dtw, bwd = om.dgrad(wd, cache, h.dout, tw)
    res = dict(idx=idx, tw=tw, out=out, dx=dx, dtw=dtw, tokens=cache["tokens"], w=w, cache=cache)
    if s.r and (tokens is None or lora_experts is not None):
        if lora_experts is not None:
            _, c2 = om.forward(w, h.x, idx, tw, experts=set(lora_experts))
            _, _, b2 = om.dgrad(wd, c2, h.dout, tw)
        else:
            c2, b2 = cache, bwd
        res["lora"] = om.lora_grad(w, c2, b2, s.E)
        res["lora_experts"] = lora_experts
    return res
