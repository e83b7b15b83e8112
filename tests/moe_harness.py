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
    import torch
    bqm = _bqm()
    E, rows, cols = w.shape
    if fmt == "nvfp4":
        q = bqm.alloc_qtensor(bqm.FMT_NVFP4, E, rows, cols, device=w.device)
        wsb = bqm.bqm_quantize_nvfp4_workspace_size(E, rows, cols, bqm.SCALE_PER_TENSOR)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=w.device)
        bqm.bqm_quantize_nvfp4(w, 1, None, q, ws)
    else:
        q = bqm.alloc_qtensor(bqm.FMT_NF4, E, rows, cols, device=w.device)
        bqm.bqm_quantize_nf4(w, q)
    return q


def poison_experts(q, experts, fmt):
    """Make the scales of the given experts decode to NaN (E4M3 0x7F / NaN absmax)."""
    import torch
    for e in experts:
        if fmt == "nvfp4":
            q.scales[e].fill_(0x7F)
        else:
            q.scales[e].fill_(float("nan"))
    torch.cuda.synchronize()


def gpu_layer(inp: synth.LayerInputs, dev, lora_scale=1.0, poison_empty=False, lora=True):
    """Forward + dgrad (+ LoRA grads) on the GPU.  Returns a dict of torch tensors."""
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
                    act_quant=int(s.act_quant), **lor)
    ws = torch.empty(max(bqm.bqm_moe_workspace_size(d), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev)
    bqm.bqm_moe_fwd(d, x, idx, tw, out, ws)
    dx = torch.empty_like(out)
    dtw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    bqm.bqm_moe_dgrad(d, dout, ws, dx, dtw)
    res = dict(idx=idx, tw=tw, out=out, dx=dx, dtw=dtw, desc=d, ws=ws)
    if s.r and lora:
        g = dict(dA_gu=torch.empty((s.E, s.r, s.H), dtype=torch.float32, device=dev),
                 dB_gu=torch.empty((s.E, 2 * s.I, s.r), dtype=torch.float32, device=dev),
                 dA_dn=torch.empty((s.E, s.r, s.I), dtype=torch.float32, device=dev),
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
        return om.MoEWeights(s.fmt, gu, dn, *lo, lora_scale=lora_scale, act_quant=s.act_quant)


def oracle_layer(h: HostInputs, lora_scale=1.0, tokens=None, lora_experts=None):
    """Oracle forward + dgrad for the chosen tokens (all if None), and LoRA grads
    for lora_experts (all experts if None and tokens is None)."""
    s = h.shape
    w = h.weights(lora_scale)
    idx, tw = orr.route(h.logits, s.k)
    out, cache = om.forward(w, h.x, idx, tw, tokens=tokens)
    dx, dtw, bwd = om.dgrad(w, cache, h.dout, tw)
    res = dict(idx=idx, tw=tw, out=out, dx=dx, dtw=dtw, tokens=cache["tokens"], w=w)
    if s.r and (tokens is None or lora_experts is not None):
        if lora_experts is not None:
            _, c2 = om.forward(w, h.x, idx, tw, experts=set(lora_experts))
            _, _, b2 = om.dgrad(w, c2, h.dout, tw)
        else:
            c2, b2 = cache, bwd
        res["lora"] = om.lora_grad(w, c2, b2, s.E)
        res["lora_experts"] = lora_experts
    return res
