"""Benchmark of the routed-expert MoE layer over NVFP4 (Four-Over-Six) experts with a bf16 LoRA.

One step = the whole layer training step on one batch of synthetic input at the
GLM-5.2 expert shape (E=256, H=6144, I=2048, top-8, T=16384 tokens, LoRA r=64):
route -> permute -> forward (gate_up GEMM + SwiGLU, down GEMM, combine) ->
dgrad through DQ(Q(W)) -> LoRA weight gradients, all in libbqm.so.  The frozen
weights are quantized once before timing (the quantizer runs per load, not per
step); its throughput on the same gate_up [256,4096,6144] and down
[256,6144,2048] stacks is measured in the same run and reported beside.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes as C
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def measured_traffic(stage):
    """HBM bytes per launch of a GEMM stage from the committed FETCH_SIZE/WRITE_SIZE
    summary, if moe.hip is still the source those counters were taken from."""
    import hashlib
    import re
    try:
        txt = open(os.path.join(ROOT, "profiles", "moe_gemm_hbm_traffic_glm.md")).read()
        blob = json.loads(re.search(r"```json\n(.*?)\n```", txt, re.S).group(1))
        src = open(os.path.join(ROOT, blob["source"]), "rb").read()
    except (OSError, AttributeError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != blob["source_sha256"]:
        return None
    st = blob["stages"].get(stage)
    return None if st is None else st["hbm_bytes"]


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch uses (one runtime per process)."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime)
        self.hip = C.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.hip.hipEventQuery.argtypes = [C.c_void_p]

    def create(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            ev = C.c_void_p()
            assert self.hip.hipEventCreate(C.byref(ev)) == 0
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        rc = self.hip.hipEventElapsedTime(C.byref(ms), a, b)
        if rc != 0:
            self.hip.hipGetLastError()        # do not leave the error for the next caller
            return None
        return ms.value

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0


def layer_flops(s):
    """Algorithmic flops of forward + dgrad (base + LoRA) and of the LoRA grads."""
    R, H, I, r = s.T * s.k, s.H, s.I, s.r
    base = 2 * R * (2 * I * H + H * I)
    lora = 2 * R * r * (H + 2 * I) + 2 * R * r * (I + H)
    return 2 * (base + lora), 2 * R * r * (2 * I + H + H + I)


def stage_flops(s):
    R, H, I, r = s.T * s.k, s.H, s.I, s.r
    return {
        "gate_up_fwd": 2 * R * 2 * I * H + 2 * R * r * 2 * I,
        "down_fwd": 2 * R * H * I + 2 * R * r * H,
        "down_dgrad": 2 * R * H * I + 2 * R * r * I,
        "gate_up_dgrad": 2 * R * 2 * I * H + 2 * R * r * H,
        "lora_a_gu": 2 * R * r * H, "lora_a_dn": 2 * R * r * I,
        "lora_b_dn": 2 * R * r * H, "lora_b_gu": 2 * R * r * 2 * I,
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, shape, experts=tuple(range(24))):
    """The oracle (float64 CPU definition) on all routed rows of a few experts, timed on
    the host.  The oracle's own quantization of the touched experts (the frozen weights
    are quantized once per load, as on the GPU) runs before the timed region and is
    reported on its own."""
    from oracle import moe as om
    from oracle import routing as orr
    from tests.moe_harness import HostInputs
    h = HostInputs(inp)
    w = h.weights()
    idx, tw = orr.route(h.logits, shape.k)
    rows = int(sum((idx == e).sum() for e in experts))
    tq = time.perf_counter()
    for e in experts:
        om.expert_matrix(w.gu, e)
        om.expert_matrix(w.dn, e)
    tq = time.perf_counter() - tq
    t0 = time.perf_counter()
    _, cache = om.forward(w, h.x, idx, tw, experts=set(experts))
    _, _, bwd = om.dgrad(w, cache, h.dout, tw)
    om.lora_grad(w, cache, bwd, shape.E)
    dt = time.perf_counter() - t0
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        threads = max(i.get("num_threads", 1) for i in threadpool_info()) or threads
    except Exception:
        pass
    per_matrix = (2 * shape.I * shape.H + shape.H * shape.I) * len(experts)
    return {"value": (rows / shape.k) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"float64 oracle forward+dgrad+LoRA grads over all {rows} routed rows of experts "
                      f"{list(experts)} (their NVFP4 weights quantized by the oracle beforehand); tokens = rows / k; "
                      f"{dt:.1f} s",
            "oracle_quantize": {"experts": len(experts), "elements": per_matrix, "s": round(tq, 2),
                                "elements_per_s": per_matrix / tq}}


def token_sweep(shape, wgu, wdn, ev, sh, tokens=(438, 1024, 2048, 4096, 8192, 16384), reps=5):
    """Layer step (route + fwd + dgrad + LoRA grads) at token counts from the pages'
    median SFT row (438) up over the same quantized experts: where the per-step read of
    the hit experts' weights gives way to MFMA time.  Each of the four grouped GEMMs
    reads one stack (gate_up or down) of every hit expert once, so a step reads the hit
    experts' NVFP4 bytes twice (10.9 GB when all 256 are hit)."""
    import dataclasses
    import torch
    import bit_quantized_moe_amd as bqm
    import synth
    dev = torch.device("cuda")
    rows = []
    for T in tokens:
        s = dataclasses.replace(shape, T=T, name=f"{shape.name}_T{T}")
        inp = synth.layer_inputs(s, device=dev, with_weights=False)
        d = bqm.MoEDesc(s.T, s.H, s.I, s.E, s.k, s.r, wgu, wdn, A_gu=inp.A_gu, B_gu=inp.B_gu, A_dn=inp.A_dn,
                        B_dn=inp.B_dn, lora_shared_a=int(s.shared_a))
        ws = torch.empty(bqm.bqm_moe_workspace_size(d), dtype=torch.uint8, device=dev)
        idx = torch.empty((T, s.k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, s.k), dtype=torch.float32, device=dev)
        out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)
        dx = torch.empty_like(out)
        dtw = torch.empty((T, s.k), dtype=torch.float32, device=dev)
        g = [torch.empty(sz, dtype=torch.float32, device=dev) for sz in
             ((s.E, s.r, s.H), (s.E, 2 * s.I, s.r), (s.E, s.r, s.I), (s.E, s.H, s.r))]

        def run():
            bqm.bqm_route(inp.logits, T, s.E, s.k, 0, idx, tw)
            bqm.bqm_moe_fwd(d, inp.x, idx, tw, out, ws)
            bqm.bqm_moe_dgrad(d, inp.dout, ws, dx, dtw)
            bqm.bqm_lora_grad(d, inp.x, inp.dout, ws, *g)

        run()
        torch.cuda.synchronize()
        e = ev.create(2)
        ev.record(e[0], sh)
        for _ in range(reps):
            run()
        ev.record(e[1], sh)
        torch.cuda.synchronize()
        ms = ev.elapsed_ms(e[0], e[1]) / reps
        hit = int(torch.unique(idx).numel())
        wbytes = 2 * hit * (2 * s.I * s.H + s.H * s.I) * (0.5 + 1 / 16)
        rows.append({"T": T, "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                     "experts_hit": hit, "weight_bytes_per_step": int(wbytes),
                     "weight_read_floor_ms": round(wbytes / (PEAK_HBM_GBS * 1e6), 4),
                     "weight_read_frac": round(wbytes / (PEAK_HBM_GBS * 1e6) / ms, 4)})
        del inp, d, ws, idx, tw, out, dx, dtw, g
        torch.cuda.empty_cache()
    return rows


def stage_bytes(s):
    """Algorithmic HBM bytes of the memory-bound stages (R = T k routed rows; the LoRA
    intermediates U and V are hi/lo bf16 pairs, 2r values per row; the LoRA weight
    gradients are written in FP32)."""
    T, R, H, I, r, E = s.T, s.T * s.k, s.H, s.I, s.r, s.E
    uv = R * 2 * r * 2
    return {
        "lora_a_gu": R * H * 2 + E * r * H * 2 + uv,
        "lora_a_dn": R * I * 2 + E * r * I * 2 + uv,
        "lora_b_dn": R * H * 2 + E * H * r * 2 + uv,
        "lora_b_gu": R * 2 * I * 2 + E * 2 * I * r * 2 + uv,
        "combine_fwd": R * H * 2 + T * H * 2 + R * 8,
        "combine_dgrad": R * H * 2 + T * H * 2 + R * 4,
        "dtopk": T * H * 2 + R * H * 2 + R * 8,
        "lora_grad": R * (2 * I + H + H + I) * 2 + 4 * uv + R * 4 + E * r * (2 * H + 3 * I) * 4,
        # per-token NVFP4 of x and a: read bf16, write codes, scales, s_dec and the bf16
        # rows of val * sb the W4A4 GEMMs multiply (one pass)
        "act_quant_x": T * H * (2 + 0.5 + 1 / 16 + 2) + T * 4,
        "act_quant_a": R * I * (2 + 0.5 + 1 / 16 + 2) + R * 4,
    }


def time_layer(s, inp, wgu, wdn, ev, sh, steps, warmup):
    """Time the layer step (route + fwd + dgrad + LoRA grads) of shape s over quantized
    experts wgu / wdn: whole-step wall time over `steps` steps after `warmup`, and each
    stage from hipEvents that the library records on the launch stream."""
    import torch
    import bit_quantized_moe_amd as bqm
    dev = torch.device("cuda")
    lora = dict(A_gu=inp.A_gu, B_gu=inp.B_gu, A_dn=inp.A_dn, B_dn=inp.B_dn) if s.r else {}
    d = bqm.MoEDesc(s.T, s.H, s.I, s.E, s.k, s.r, wgu, wdn, act_quant=int(s.act_quant),
                    lora_shared_a=int(s.shared_a), **lora)
    ws = torch.empty(bqm.bqm_moe_workspace_size(d), dtype=torch.uint8, device=dev)
    idx = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
    tw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(out)
    dtw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    ea = () if s.shared_a else (s.E,)
    g = [torch.empty(sz, dtype=torch.float32, device=dev) for sz in
         (ea + (s.r, s.H), (s.E, 2 * s.I, s.r), ea + (s.r, s.I), (s.E, s.H, s.r))] if s.r else [None] * 4

    def step(events=None):
        d.stage_events = C.addressof(events) if events is not None else None
        bqm.bqm_route(inp.logits, s.T, s.E, s.k, 0, idx, tw)
        bqm.bqm_moe_fwd(d, inp.x, idx, tw, out, ws)
        bqm.bqm_moe_dgrad(d, inp.dout, ws, dx, dtw)
        if s.r:
            bqm.bqm_lora_grad(d, inp.x, inp.dout, ws, *g)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [ev.create(2 * bqm.STAGE_COUNT) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps

    stages = {}
    for si, name in enumerate(bqm.STAGES):
        if name.startswith("act_quant") and not s.act_quant:
            continue
        v = [ev.elapsed_ms(e[2 * si], e[2 * si + 1]) for e in evs]
        v = [x for x in v if x is not None]
        if v:
            stages[name] = sum(v) / len(v)
    sf = stage_flops(s)
    sb = stage_bytes(s)
    gemms = {k: v for k, v in stages.items() if k in ("gate_up_fwd", "down_fwd", "down_dgrad", "gate_up_dgrad")}
    dom = max(gemms, key=gemms.get)
    roof = {}
    for k, v in stages.items():
        if k in gemms:
            roof[k] = {"bound": "mfma", "frac": round(sf[k] / (v * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        elif k in sb:
            roof[k] = {"bound": "hbm", "GB/s": round(sb[k] / (v * 1e-3) / 1e9, 1),
                       "frac": round(sb[k] / (v * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    fl, fl_lora = layer_flops(s)
    res = {
        "tokens_per_s": s.T / (ms * 1e-3), "ms_per_step": ms,
        "fwd_dgrad_tokens_per_s": s.T / (sum(v for k, v in stages.items() if k != "lora_grad") * 1e-3),
        "layer_tflops": (fl + fl_lora) / (ms * 1e-3) / 1e12,
        "dominant_gemm": dom, "dominant_ms": gemms[dom],
        "dominant_tflops": sf[dom] / (gemms[dom] * 1e-3) / 1e12,
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "stage_roofline": roof,
    }
    del d, ws, idx, tw, out, dx, dtw, g
    torch.cuda.empty_cache()
    return res


def decode_sweep(shape, wgu, wdn, ev, sh, tokens=(1, 8, 32, 64, 256), reps=20, warmup=3, graph=True):
    """Decode-shaped forward (route + moe_fwd only) at a few tokens over the same
    quantized experts and LoRA: the time against reading each hit expert's NVFP4
    weights (codes + E4M3 scales of gate_up and down) once."""
    import dataclasses
    import torch
    import bit_quantized_moe_amd as bqm
    import synth
    dev = torch.device("cuda")
    per_expert = (2 * shape.I * shape.H + shape.H * shape.I) * (0.5 + 1 / 16)
    rows = []
    for T in tokens:
        s = dataclasses.replace(shape, T=T, name=f"{shape.name}_decode_T{T}")
        inp = synth.layer_inputs(s, device=dev, with_weights=False)
        d = bqm.MoEDesc(s.T, s.H, s.I, s.E, s.k, s.r, wgu, wdn, A_gu=inp.A_gu, B_gu=inp.B_gu, A_dn=inp.A_dn,
                        B_dn=inp.B_dn, lora_shared_a=int(s.shared_a))
        ws = torch.empty(bqm.bqm_moe_workspace_size(d), dtype=torch.uint8, device=dev)
        idx = torch.empty((T, s.k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, s.k), dtype=torch.float32, device=dev)
        out = torch.empty((T, s.H), dtype=torch.bfloat16, device=dev)

        def run():
            bqm.bqm_route(inp.logits, T, s.E, s.k, 0, idx, tw)
            bqm.bqm_moe_fwd(d, inp.x, idx, tw, out, ws)

        for _ in range(warmup):
            run()
        ms = time_calls(ev, sh, run, reps)
        # the same forward captured once in a HIP graph and replayed (no launch work on the
        # host per forward): captured on a side stream after warmup, replayed on this one
        gms = None
        if graph:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                run()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run()
            torch.cuda.synchronize()
            gms = time_calls(ev, sh, g.replay, reps)
            del g
        hit = int(torch.unique(idx).numel())
        wbytes = hit * per_expert
        rows.append({"T": T, "ms_per_forward": round(ms, 4),
                     "ms_per_forward_graph_replay": None if gms is None else round(gms, 4), "experts_hit": hit,
                     "hit_weight_bytes": int(wbytes), "weight_read_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
                     "weight_read_frac": round(wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
        del inp, d, ws, idx, tw, out
        torch.cuda.empty_cache()
    return rows


def colwise_comparison(s, inp, wgu, wdn, ev, sh, reps=5):
    """The two-copy scheme as a comparison: the dgrad over a second, columnwise NVFP4
    quantization (Q(W^T), read K-major) against the transposed read of the single
    rowwise copy, at the same layer and routing.  Reports both dgrads' GEMM times, the
    weight bytes each scheme holds, and how far the two dX results are apart (the
    columnwise copy dequantizes to different values)."""
    import torch
    import bit_quantized_moe_amd as bqm
    dev = torch.device("cuda")
    t = inp.w_gu.transpose(1, 2).contiguous()
    cgu = bqm.quantize_stack(t, "nvfp4")
    del t
    t = inp.w_dn.transpose(1, 2).contiguous()
    cdn = bqm.quantize_stack(t, "nvfp4")
    del t
    torch.cuda.empty_cache()
    d = bqm.MoEDesc(s.T, s.H, s.I, s.E, s.k, s.r, wgu, wdn, A_gu=inp.A_gu, B_gu=inp.B_gu, A_dn=inp.A_dn,
                    B_dn=inp.B_dn)
    ws = torch.empty(bqm.bqm_moe_workspace_size(d), dtype=torch.uint8, device=dev)
    idx = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
    tw = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev)
    dx_row, dx_col = torch.empty_like(out), torch.empty_like(out)
    bqm.bqm_route(inp.logits, s.T, s.E, s.k, 0, idx, tw)
    bqm.bqm_moe_fwd(d, inp.x, idx, tw, out, ws)

    def stages(fn):
        res = {}
        for it in range(reps + 1):
            e = ev.create(2 * bqm.STAGE_COUNT)
            d.stage_events = C.addressof(e)
            fn()
            torch.cuda.synchronize()
            if it:
                for si, n in enumerate(bqm.STAGES):
                    if n in ("down_dgrad", "gate_up_dgrad"):
                        res.setdefault(n, []).append(ev.elapsed_ms(e[2 * si], e[2 * si + 1]))
        d.stage_events = None
        return {k: round(sum(v) / len(v), 4) for k, v in res.items()}

    row = stages(lambda: bqm.bqm_moe_dgrad(d, inp.dout, ws, dx_row, None))
    col = stages(lambda: bqm.bqm_moe_dgrad_colwise(d, cgu, cdn, inp.dout, ws, dx_col, None))
    diff = float((dx_col.float() - dx_row.float()).norm() / dx_row.float().norm())
    wbytes = sum(q.codes.numel() + q.scales.numel() + q.s_dec.numel() * 4 for q in (wgu, wdn))
    res = {"workload": "glm5.2 layer dgrad (T=16384), nvfp4 weights", "rowwise_transposed_read_ms": row,
           "columnwise_copy_ms": col, "weight_bytes_one_copy": wbytes, "weight_bytes_two_copies": 2 * wbytes,
           "dx_rel_diff_between_schemes": diff}
    del cgu, cdn, d, ws, idx, tw, out, dx_row, dx_col
    torch.cuda.empty_cache()
    return res


def time_calls(ev, sh, fn, reps=3):
    """Mean hipEvent time of fn() over reps calls after one untimed call."""
    import torch
    fn()
    torch.cuda.synchronize()
    e = ev.create(2)
    ev.record(e[0], sh)
    for _ in range(reps):
        fn()
    ev.record(e[1], sh)
    torch.cuda.synchronize()
    return ev.elapsed_ms(e[0], e[1]) / reps


def row_tiles(logits, s):
    """256-row tiles of the grouped GEMMs under a routing: the sum over experts of
    ceil(rows / 256), with the top-k of the logits as the library's router picks them."""
    import torch
    import bit_quantized_moe_amd as bqm
    idx = torch.empty((s.T, s.k), dtype=torch.int32, device=logits.device)
    tw = torch.empty((s.T, s.k), dtype=torch.float32, device=logits.device)
    bqm.bqm_route(logits, s.T, s.E, s.k, 0, idx, tw)
    n = torch.bincount(idx.reshape(-1).long(), minlength=s.E)
    return {"tiles": int(((n + 255) // 256).sum()), "rows_min": int(n.min()), "rows_max": int(n.max())}


def config_block(s, res, weights):
    return {"workload": s.name, "E": s.E, "H": s.H, "I": s.I, "k": s.k, "T": s.T, "r": s.r,
            "weights": weights, "act_quant": bool(s.act_quant), "routing": s.logits,
            "tokens_per_s": res["tokens_per_s"], "ms_per_step": res["ms_per_step"],
            "fwd_dgrad_tokens_per_s": res["fwd_dgrad_tokens_per_s"], "layer_tflops": res["layer_tflops"],
            "dominant_gemm": res["dominant_gemm"],
            "dominant_frac": res["dominant_tflops"] / PEAK_BF16_TFLOPS,
            "stages_ms": res["stages_ms"], "stage_roofline": res["stage_roofline"]}


def summarize_counters(root, min_us=300.0):
    """Per-kernel table from a rocprofv3 --pmc --kernel-trace --output-format csv run under
    root: launches, average duration, shader clock (GRBM_GUI_ACTIVE summed over the 8
    XCDs / duration / 8), the MFMA-busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the four
    SIMDs of every busy CU cycle) and each counter's average per launch.  Launches
    shorter than min_us are left out (the counters' start and stop dominate them)."""
    import collections
    import csv
    import glob
    import re
    dur, name = {}, {}
    for f in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            name[r["Dispatch_Id"]] = re.sub(r"\(anonymous namespace\)::", "", r["Kernel_Name"])
    ctr = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv*"), recursive=True):
        for r in csv.DictReader(open(f)):
            ctr[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            if r["Dispatch_Id"] not in dur:  # no kernel trace kept: the counter rows carry the times
                dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                name[r["Dispatch_Id"]] = re.sub(r"\(anonymous namespace\)::", "", r["Kernel_Name"])
    agg = collections.defaultdict(lambda: [0, 0.0, collections.defaultdict(float)])
    for d, t in dur.items():
        if t < min_us * 1e3 or d not in ctr:
            continue
        a = agg[name[d]]
        a[0] += 1
        a[1] += t
        for k, v in ctr[d].items():
            a[2][k] += v
    rows = []
    for n, (c, t, cs) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        row = {"kernel": n.split("(")[0] if "bqm" in n else n[:90], "launches": c, "avg_us": round(t / c / 1e3, 1)}
        if "GRBM_GUI_ACTIVE" in cs:
            row["ghz"] = round(cs["GRBM_GUI_ACTIVE"] / t / 8, 3)
        if "SQ_BUSY_CU_CYCLES" in cs and "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
            row["mfma_busy"] = round(cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * cs["SQ_BUSY_CU_CYCLES"]), 3)
        if "SQ_LDS_BANK_CONFLICT" in cs and cs.get("SQ_LDS_IDX_ACTIVE"):
            row["lds_bank_conflict_frac"] = round(cs["SQ_LDS_BANK_CONFLICT"] / cs["SQ_LDS_IDX_ACTIVE"], 3)
        if cs.get("SQ_INSTS_MFMA"):
            row["valu_per_mfma"] = round(cs["SQ_INSTS_VALU"] / cs["SQ_INSTS_MFMA"], 2) if "SQ_INSTS_VALU" in cs else None
        for k in sorted(cs):
            row[k] = cs[k] / c
        rows.append(row)
    return rows


def library_gemm_reference(ev, sh):
    """bf16 GEMMs of the vendor library (through torch) at the GLM gate_up shape, for
    context beside the grouped 4-bit GEMM: one GEMM over all 131072 routed rows
    [131072, 6144] x [6144, 4096] (one weight for all rows), and the per-expert batch
    [256][512, 6144] x [256][6144, 4096] with bf16 weights (12.9 GB of them)."""
    import torch
    dev = torch.device("cuda")
    fl = 2 * 131072 * 6144 * 4096
    res = {}
    a = torch.randn(256, 512, 6144, device=dev, dtype=torch.bfloat16)
    w = torch.randn(4096, 6144, device=dev, dtype=torch.bfloat16)
    a2 = a.view(-1, 6144)
    ms = time_calls(ev, sh, lambda: torch.nn.functional.linear(a2, w), 5)
    res["one_gemm_131072x6144x4096"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                        "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    del w
    b = torch.randn(256, 6144, 4096, device=dev, dtype=torch.bfloat16)
    ms = time_calls(ev, sh, lambda: torch.bmm(a, b), 5)
    res["batched_256x512x6144x4096"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                        "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    del a, a2, b
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="only the GLM NVFP4 layer step (and the quantizer unless --no-quantizer): no NF4, "
                         "W4A4, format-conversion or token-sweep figures")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the layer step at smaller token counts (the token sweep)")
    ap.add_argument("--workload", choices=["glm", "glm_nf4", "glm_nf4_nested", "qwen"],
                    help="only the layer step of this workload (for profiling): prints its timings, no bench line")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the per-kernel table of a rocprofv3 --pmc --kernel-trace csv run under DIR, no GPU")
    ap.add_argument("--decode-tokens", type=int, metavar="T",
                    help="only the decode-shaped forward (route + moe_fwd) of the GLM shape at T tokens, "
                         "`steps` times after `warmup` (for profiling): prints its timings, no bench line")
    ap.add_argument("--library-reference", action="store_true",
                    help="only time the vendor library's bf16 GEMMs at the GLM gate_up shape")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.summarize_counters:
        for row in summarize_counters(args.summarize_counters):
            print(json.dumps(row))
        return
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_call": 1 << 30, "calls": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the layer runs and is timed on a single MI355X. "
              "There is no multi-GPU path (expert parallelism would add one all-to-all of the "
              "routed rows each way around these same kernels).", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_moe_amd as bqm
    import synth

    dev = torch.device("cuda")
    bqm.load()
    if args.library_reference:
        print(json.dumps(library_gemm_reference(HipEvents(), torch.cuda.current_stream().cuda_stream)), flush=True)
        return
    if args.decode_tokens:
        s1 = synth.GLM
        inp1 = synth.layer_inputs(s1, device=dev)
        wgu1 = bqm.quantize_stack(inp1.w_gu, s1.fmt)
        wdn1 = bqm.quantize_stack(inp1.w_dn, s1.fmt)
        del inp1
        torch.cuda.empty_cache()
        ev = HipEvents()
        rows = decode_sweep(s1, wgu1, wdn1, ev, torch.cuda.current_stream().cuda_stream,
                            tokens=(args.decode_tokens,), reps=args.steps, warmup=args.warmup)
        print(json.dumps({"workload": "glm5.2 decode forward", **rows[0]}), flush=True)
        return
    if args.workload:
        ws_ = {"glm": synth.GLM, "glm_nf4": synth.GLM_NF4, "qwen": synth.QWEN,
               "glm_nf4_nested": dataclasses.replace(synth.GLM_NF4, fmt="nf4_nested", name="glm_nf4_nested")}
        s1 = ws_[args.workload]
        inp1 = synth.layer_inputs(s1, device=dev)
        wgu1 = bqm.quantize_stack(inp1.w_gu, s1.fmt)
        wdn1 = bqm.quantize_stack(inp1.w_dn, s1.fmt)
        inp1.w_gu = inp1.w_dn = None
        torch.cuda.empty_cache()
        r1 = time_layer(s1, inp1, wgu1, wdn1, HipEvents(), torch.cuda.current_stream().cuda_stream,
                        args.steps, args.warmup)
        print(json.dumps({"workload": s1.name, **r1}), flush=True)
        return
    shape = synth.GLM
    s = shape
    inp = synth.layer_inputs(shape, device=dev)
    ev = HipEvents()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    # a plain device-to-device copy of 2 GiB: the HBM rate reachable in practice, beside the 8 TB/s spec
    cbuf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(cbuf)
    copy_ms = time_calls(ev, sh, lambda: cdst.copy_(cbuf), 5)
    hbm_copy = {"bytes_moved": 2 * (1 << 31), "ms": copy_ms, "GB/s": 2 * (1 << 31) / copy_ms / 1e6,
                "frac_of_spec": 2 * (1 << 31) / copy_ms / 1e6 / PEAK_HBM_GBS}
    del cbuf, cdst
    torch.cuda.empty_cache()
    n_el = s.E * (2 * s.I * s.H + s.H * s.I)
    conv_bytes = n_el * (2 + 0.5 + 1 / 16)    # bf16 <-> 4-bit codes + 1 scale byte (or 1/4 float) per 16

    # --- quantizer (per load): gate_up + down stacks, timed with events ---
    quant = None
    formats = {}
    if not args.no_quantizer:
        qgu = bqm.alloc_qtensor(bqm.FMT_NVFP4, s.E, 2 * s.I, s.H, device=dev)
        qdn = bqm.alloc_qtensor(bqm.FMT_NVFP4, s.E, s.H, s.I, device=dev)
        wsq = torch.empty(bqm.bqm_quantize_nvfp4_workspace_size(s.E, 2 * s.I, s.H, 0), dtype=torch.uint8,
                          device=dev)
        def time_quant(sd_gu, sd_dn):
            times = []
            for it in range(4):
                e = ev.create(2)
                ev.record(e[0], sh)
                bqm.bqm_quantize_nvfp4(inp.w_gu, 1, sd_gu, qgu, wsq)
                bqm.bqm_quantize_nvfp4(inp.w_dn, 1, sd_dn, qdn, wsq)
                ev.record(e[1], sh)
                torch.cuda.synchronize()
                if it:
                    times.append(ev.elapsed_ms(e[0], e[1]))
            return sum(times) / len(times)

        qms = time_quant(None, None)
        # the same quantization with the per-tensor scales handed in (frozen weights
        # re-quantized with known scales): one read of the input instead of two
        sd_gu, sd_dn = qgu.s_dec.clone(), qdn.s_dec.clone()
        gms = time_quant(sd_gu, sd_dn)
        quant = {"workload": "gate_up [256,4096,6144] + down [256,6144,2048] bf16 -> NVFP4 4/6",
                 "ms": qms, "GB/s": conv_bytes / qms / 1e6, "hbm_frac": conv_bytes / qms / 1e6 / PEAK_HBM_GBS,
                 "algorithmic_bytes": conv_bytes,
                 "note": "per-tensor scale from the stack's own amax: the input is read twice (amax pass, "
                         "then quantize pass); algorithmic bytes count one read",
                 # the bytes this mode has to move: the bf16 stacks twice, the codes and scales once
                 "two_read_bytes": conv_bytes + n_el * 2,
                 "two_read_hbm_frac": (conv_bytes + n_el * 2) / qms / 1e6 / PEAK_HBM_GBS,
                 "given_scale": {"ms": gms, "GB/s": conv_bytes / gms / 1e6,
                                 "hbm_frac": conv_bytes / gms / 1e6 / PEAK_HBM_GBS}}
        wgu, wdn = qgu, qdn
        del wsq
    else:
        wgu = bqm.quantize_stack(inp.w_gu, "nvfp4")
        wdn = bqm.quantize_stack(inp.w_dn, "nvfp4")

    res = time_layer(s, inp, wgu, wdn, ev, sh, args.steps, args.warmup)
    sf = stage_flops(s)
    dom = res["dominant_gemm"]
    ach = res["dominant_tflops"]
    result = {
        "metric": "NVFP4 MoE layer fwd+dgrad tokens/s (GLM-5.2 shape); quantizer GB/s",
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "glm5.2-moe-layer-train-step", "E": s.E, "H": s.H, "I": s.I, "k": s.k,
                   "T": s.T, "r": s.r, "weights": "nvfp4-4over6-rowwise", "step": "route+fwd+dgrad+lora_grad",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom),
                     "algorithmic_flop_per_launch": sf[dom], "launch_ms": res["dominant_ms"]},
        "layer_tflops": res["layer_tflops"],
        "fwd_dgrad_tokens_per_s": res["fwd_dgrad_tokens_per_s"],
        "stages_ms": res["stages_ms"],
        "stage_roofline": res["stage_roofline"],
        "quantizer": quant,
        "hbm_copy": hbm_copy,
    }

    if not args.main_only:
        # --- format conversions on the same stacks: NVFP4 dequantize, NF4 quantize / dequantize ---
        ybuf = torch.empty_like(inp.w_gu)
        ydn = ybuf.view(-1)[: inp.w_dn.numel()].view(inp.w_dn.shape)
        if not args.no_quantizer:
            ms = time_calls(ev, sh, lambda: (bqm.bqm_dequantize(wgu, ybuf), bqm.bqm_dequantize(wdn, ydn)))
            formats["nvfp4_dequantize"] = {"ms": ms, "GB/s": conv_bytes / ms / 1e6,
                                           "hbm_frac": conv_bytes / ms / 1e6 / PEAK_HBM_GBS}
        if not args.no_quantizer:
            # the strict FP32 reference form of the 4/6 choice (candidates scaled back up and
            # compared with the original values) on the same stacks, and how often its choice
            # agrees with the scaled-domain form used everywhere else
            sgu = bqm.alloc_qtensor(bqm.FMT_NVFP4, s.E, 2 * s.I, s.H, device=dev)
            sdn = bqm.alloc_qtensor(bqm.FMT_NVFP4, s.E, s.H, s.I, device=dev)
            wsq2 = torch.empty(bqm.bqm_quantize_nvfp4_workspace_size(s.E, 2 * s.I, s.H, 0), dtype=torch.uint8,
                               device=dev)
            ms = time_calls(ev, sh, lambda: (bqm.bqm_quantize_nvfp4(inp.w_gu, 2, None, sgu, wsq2),
                                             bqm.bqm_quantize_nvfp4(inp.w_dn, 2, None, sdn, wsq2)))
            nblk = sgu.scales.numel() + sdn.scales.numel()
            same = int((sgu.scales == wgu.scales).sum()) + int((sdn.scales == wdn.scales).sum())
            formats["nvfp4_quantize_strict_4over6"] = {
                "ms": ms, "GB/s": conv_bytes / ms / 1e6, "hbm_frac": conv_bytes / ms / 1e6 / PEAK_HBM_GBS,
                "blocks": nblk, "same_choice_as_scaled_form": same / nblk}
            del sgu, sdn, wsq2
            torch.cuda.empty_cache()
        ngu = bqm.alloc_qtensor(bqm.FMT_NF4, s.E, 2 * s.I, s.H, device=dev)
        ndn = bqm.alloc_qtensor(bqm.FMT_NF4, s.E, s.H, s.I, device=dev)
        nf4_bytes = n_el * (2 + 0.5 + 4 / 64)
        ms = time_calls(ev, sh, lambda: (bqm.bqm_quantize_nf4(inp.w_gu, ngu), bqm.bqm_quantize_nf4(inp.w_dn, ndn)))
        formats["nf4_quantize"] = {"ms": ms, "GB/s": nf4_bytes / ms / 1e6,
                                   "hbm_frac": nf4_bytes / ms / 1e6 / PEAK_HBM_GBS}
        ms = time_calls(ev, sh, lambda: (bqm.bqm_dequantize(ngu, ybuf), bqm.bqm_dequantize(ndn, ydn)))
        formats["nf4_dequantize"] = {"ms": ms, "GB/s": nf4_bytes / ms / 1e6,
                                     "hbm_frac": nf4_bytes / ms / 1e6 / PEAK_HBM_GBS}
        # nested (double-quantized) absmax: the nesting pass over the FP32 absmax, the
        # dequantize from the nested form, and the storage of the two stacks
        mgu = bqm.alloc_qtensor(bqm.FMT_NF4, s.E, 2 * s.I, s.H, device=dev, nested=1)
        mdn = bqm.alloc_qtensor(bqm.FMT_NF4, s.E, s.H, s.I, device=dev, nested=1)
        mgu.codes, mdn.codes = ngu.codes, ndn.codes
        ms = time_calls(ev, sh, lambda: (bqm.bqm_nf4_nest(ngu, mgu), bqm.bqm_nf4_nest(ndn, mdn)))
        nest_bytes = n_el * (4 / 64 + 1 / 64) + 4 * (mgu.s_dec.numel() + mdn.s_dec.numel())
        nested_stack_bytes = n_el // 2 + n_el // 64 + 4 * (mgu.s_dec.numel() + mdn.s_dec.numel())
        formats["nf4_nest"] = {"ms": ms, "GB/s": nest_bytes / ms / 1e6,
                               "hbm_frac": nest_bytes / ms / 1e6 / PEAK_HBM_GBS,
                               "stack_bytes_plain": int(n_el // 2 + n_el // 64 * 4),
                               "stack_bytes_nested": int(nested_stack_bytes),
                               "bits_per_weight_nested": 8 * nested_stack_bytes / n_el}
        nfn_bytes = n_el * (2 + 0.5 + 1 / 64)
        ms = time_calls(ev, sh, lambda: (bqm.bqm_dequantize(mgu, ybuf), bqm.bqm_dequantize(mdn, ydn)))
        formats["nf4_nested_dequantize"] = {"ms": ms, "GB/s": nfn_bytes / ms / 1e6,
                                            "hbm_frac": nfn_bytes / ms / 1e6 / PEAK_HBM_GBS}
        formats["workload"] = "gate_up [256,4096,6144] + down [256,6144,2048]; bytes = 2 (bf16) + 0.5 (codes) " \
                              "+ scale bytes per element"
        result["formats"] = formats
        del ybuf, ydn
        torch.cuda.empty_cache()

        # --- the other layer workloads: GLM shape over NF4 experts with skewed routing
        # (16 experts empty), and the Qwen3-30B-A3B shape with NVFP4 activations (W4A4) ---
        others = {}
        s5 = synth.GLM_NF4
        inp5 = synth.layer_inputs(s5, device=dev, with_weights=False)
        r5 = time_layer(s5, inp5, ngu, ndn, ev, sh, max(3, args.steps // 2), 2)
        others["glm_nf4_zipf"] = config_block(s5, r5, "nf4-blocksize64")
        s5n = dataclasses.replace(s5, fmt="nf4_nested", name="glm_nf4_nested_zipf")
        r5n = time_layer(s5n, inp5, mgu, mdn, ev, sh, max(3, args.steps // 2), 2)
        others["glm_nf4_nested_zipf"] = config_block(s5n, r5n, "nf4-blocksize64, double-quantized absmax")
        del inp5, ngu, ndn, mgu, mdn
        torch.cuda.empty_cache()
        s3 = synth.QWEN
        inp3 = synth.layer_inputs(s3, device=dev)
        q3gu = bqm.quantize_stack(inp3.w_gu, "nvfp4")
        q3dn = bqm.quantize_stack(inp3.w_dn, "nvfp4")
        r3 = time_layer(s3, inp3, q3gu, q3dn, ev, sh, max(3, args.steps), 2)
        others["qwen3_30b_a3b_w4a4"] = config_block(s3, r3, "nvfp4-4over6-rowwise, activations nvfp4 per token")
        del inp3, q3gu, q3dn
        torch.cuda.empty_cache()
        # the tiny workload (8 experts, 64 tokens): every launch is a few microseconds
        s1t = synth.TINY
        inp1t = synth.layer_inputs(s1t, device=dev)
        q1gu = bqm.quantize_stack(inp1t.w_gu, s1t.fmt)
        q1dn = bqm.quantize_stack(inp1t.w_dn, s1t.fmt)
        r1t = time_layer(s1t, inp1t, q1gu, q1dn, ev, sh, max(10, args.steps), 3)
        others["tiny"] = config_block(s1t, r1t, "nvfp4-4over6-rowwise")
        del inp1t, q1gu, q1dn
        # the GLM layer with the adapter layout of the GLM page (one LoRA-A shared by all
        # experts, per-expert LoRA-B) over the same NVFP4 experts
        s_sh = dataclasses.replace(shape, shared_a=True, name="glm_shared_lora_a")
        inp_sh = synth.layer_inputs(s_sh, device=dev, with_weights=False)
        r_sh = time_layer(s_sh, inp_sh, wgu, wdn, ev, sh, max(3, args.steps // 2), 2)
        others["glm_nvfp4_shared_lora_a"] = config_block(s_sh, r_sh, "nvfp4-4over6-rowwise, one LoRA-A for all "
                                                                     "experts, per-expert LoRA-B")
        del inp_sh
        torch.cuda.empty_cache()
        # the same GLM layer with every expert at exactly R / E rows: the synthetic routing's
        # spread (446-579 rows per expert at this shape) leaves a mostly empty third 256-row
        # tile on every expert above 512 rows, each a full pass over its weights
        s_bal = dataclasses.replace(shape, logits="balanced", name="glm_balanced_routing")
        inp_bal = synth.layer_inputs(s_bal, device=dev, with_weights=False)
        r_bal = time_layer(s_bal, inp_bal, wgu, wdn, ev, sh, max(3, args.steps // 2), 2)
        others["glm_nvfp4_balanced_routing"] = config_block(s_bal, r_bal, "nvfp4-4over6-rowwise")
        others["glm_nvfp4_balanced_routing"]["row_tiles_256"] = {
            "synthetic_routing": row_tiles(inp.logits, shape), "balanced_routing": row_tiles(inp_bal.logits, s_bal)}
        del inp_bal
        torch.cuda.empty_cache()
        result["other_configs"] = others
        # the two-copy scheme (a columnwise second quantization for the dgrad) as a comparison
        result["columnwise_dgrad_comparison"] = colwise_comparison(s, inp, wgu, wdn, ev, sh)
        # the vendor library's bf16 GEMMs at the gate_up shape, for context
        result["library_bf16_gemm_reference"] = library_gemm_reference(ev, sh)
        # decode-shaped forward over the GLM experts (serving side: weight-read-bound)
        result["decode_forward"] = {"workload": "glm5.2 shape, forward only (route + moe_fwd), nvfp4 weights, "
                                                "LoRA r=64", "rows": decode_sweep(shape, wgu, wdn, ev, sh),
                                    "rows_shared_lora_a": decode_sweep(dataclasses.replace(shape, shared_a=True),
                                                                       wgu, wdn, ev, sh)}

    if not args.no_sweep and not args.main_only:
        torch.cuda.empty_cache()
        result["token_sweep"] = token_sweep(shape, wgu, wdn, ev, sh)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, shape)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
