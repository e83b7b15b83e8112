"""GPU parity of the MoE layer (forward, dgrad through DQ(Q(W)), LoRA gradients)
against the float64 oracle, on small layers that span several tiles with ragged
expert segments, on the tiny workload, and sampled at the full workload sizes."""
import dataclasses

import numpy as np
import pytest

import synth
from tests.gpu_util import assert_close, gpu, log, np_f32
from tests.moe_harness import HostInputs, gpu_layer, oracle_layer, resolve_w4a4_alternatives

pytestmark = pytest.mark.gpu


def small(name, **kw):
    base = dict(E=16, H=512, I=256, k=4, T=300, r=16, seed=7, outliers=True)
    base.update(kw)
    return synth.Shape(name, **base)


def compare_full(shape, lora_scale=1.0, poison_empty=False, colwise=False):
    dev = gpu()
    log(f"layer {shape}" + (" (dgrad over columnwise copies)" if colwise else ""))
    inp = synth.layer_inputs(shape, device="cpu")
    g = gpu_layer(inp, dev, lora_scale=lora_scale, poison_empty=poison_empty, colwise=colwise)
    h = HostInputs(inp)
    o = oracle_layer(h, lora_scale=lora_scale, colwise=colwise)
    assert (g["idx"].cpu().numpy() == o["idx"]).all(), "routing indices"
    n_alt = resolve_w4a4_alternatives(np_f32(g["out"]), None, o, h)
    errs = {}
    errs["out"] = assert_close(np_f32(g["out"]), o["out"], "out")
    errs["dx"] = assert_close(np_f32(g["dx"]), o["dx"], "dx")
    errs["dtw"] = assert_close(g["dtw"].cpu().numpy(), o["dtw"], "dtopk_w")
    if shape.r:
        for name, ref in zip(("dA_gu", "dB_gu", "dA_dn", "dB_dn"), o["lora"]):
            got = g[name].cpu().numpy()
            errs[name] = assert_close(got, ref, name)
            if shape.shared_a and name.startswith("dA"):
                continue  # one shared matrix, not a per-expert stack
            hit = np.zeros(shape.E, bool)
            hit[o["idx"].reshape(-1)] = True
            assert (got[~hit] == 0).all(), f"{name}: experts without rows must get zeros"
    log("  " + ", ".join(f"{k}={v[0]:.2e}/{v[1]:.2e}" for k, v in errs.items()) + f" (w4a4 rows with a valid alternative: {n_alt})")
    return g, o


def test_small_nvfp4_lora():
    compare_full(small("small"), lora_scale=0.5)


def test_small_nvfp4_partial_tiles():
    # H and I multiples of 64 but not of 256: partial column tiles in all four GEMMs
    # (gate_up N = 2I = 384, down N = H = 320, dgrad N = I = 192 and H = 320) and
    # odd K-step counts (5, 3, 5, 6)
    compare_full(small("small_odd", H=320, I=192, T=260, E=12))


def test_small_nvfp4_colwise_dgrad():
    # the two-copy comparison variant: the dgrad over Q(W^T) read K-major, against the
    # oracle's DQ(Q(W^T))^T; ragged tiles and partial column tiles included
    compare_full(small("small_col", H=320, I=192, T=260, E=12), lora_scale=0.5, colwise=True)
    compare_full(small("small_col2"), colwise=True)


def test_small_nvfp4_no_lora():
    compare_full(small("small_r0", r=0, T=97, k=2))


def test_small_w4a4():
    compare_full(small("small_w4a4", act_quant=True, H=768, I=384))


def test_small_nf4_skewed_with_empty_experts():
    g, o = compare_full(small("small_nf4", fmt="nf4", logits="zipf", E=64, T=200, k=4, r=8), poison_empty=True)
    counts = np.bincount(o["idx"].reshape(-1), minlength=64)
    assert (counts == 0).sum() >= 16


def test_small_nf4_nested_absmax_skewed_with_empty_experts():
    # NF4 weights with the double-quantized absmax (the GEMMs rebuild absmax' from
    # the E4M3 code, the group scale and the offset); empty experts poisoned
    g, o = compare_full(small("small_nf4n", fmt="nf4_nested", logits="zipf", E=64, T=200, k=4, r=8),
                        poison_empty=True)
    assert (np.bincount(o["idx"].reshape(-1), minlength=64) == 0).sum() >= 16


def test_nvfp4_routed_only_poisoned_experts():
    shape = small("small_zipf", logits="zipf", E=48, T=128, k=4, r=8)
    g, o = compare_full(shape, poison_empty=True)
    assert np.isfinite(np_f32(g["out"])).all() and np.isfinite(np_f32(g["dx"])).all()


def test_small_shared_lora_a():
    # one LoRA-A for all experts, its gradients summed over 12 parts of one expert
    # each; partial column tiles as in the ragged case above
    compare_full(small("small_sh", H=320, I=192, T=600, E=12, shared_a=True), lora_scale=0.5)


def test_small_shared_lora_a_nf4_w4a4_colwise():
    # the same layout on the NF4 kernels with skewed routing and empty experts (64
    # experts in parts of one, some empty), on the W4A4 path and on the columnwise dgrad
    g, o = compare_full(small("small_sh_nf4", fmt="nf4", logits="zipf", E=64, T=700, k=4, r=8, shared_a=True),
                        poison_empty=True)
    assert (np.bincount(o["idx"].reshape(-1), minlength=64) == 0).sum() >= 16
    compare_full(small("small_sh_w4a4", act_quant=True, H=768, I=384, T=600, shared_a=True))
    # 96 experts: parts of one or two experts
    compare_full(small("small_sh_col", shared_a=True, E=96, T=400), colwise=True)


def test_small_batches():
    # decode-sized batches (at most 32 routed rows per expert on average: the forward and
    # the NVFP4 dgrad run the 64-row tile configuration), where most row tiles hold one or two valid
    # 32-row tiles: T = 8 over 64 experts with k = 8; partial column tiles at T = 40;
    # 100 rows per expert (the 256-row tiles again); T = 256 with the shared-A LoRA;
    # NVFP4 activations; LoRA rank 72 (masked K tail of the up-projection segment)
    compare_full(small("dec8", T=8, E=64, k=8, r=16), lora_scale=0.5)
    compare_full(small("dec_odd", H=320, I=192, T=40, E=12))
    compare_full(small("dec_rows", T=200, E=4, k=2, r=8))
    compare_full(small("dec256", T=256, E=32, k=4, shared_a=True))
    compare_full(small("dec_w4a4", act_quant=True, H=768, I=384, T=64, E=16, k=4))
    compare_full(small("dec_r72", r=72, T=60, E=16, k=4), lora_scale=0.5)


def test_streaming_forward():
    # decode-sized batches with a few routed rows per expert on average (T k <= 2 E for
    # gate_up, <= 4 E for down): the forward streams the weights, up to 16 rows of an
    # expert per pass.  T = 1; zipf routing over 128 experts (experts above 16 rows: several
    # passes; the 16 empty experts NaN-poisoned, never read); one expert with about 70
    # rows (two 64-row tiles); H = 320, I = 192 (a half 128-deep block ends each K);
    # NVFP4 activations; LoRA rank 72 with the shared A; no LoRA; H = I = 64 (one half
    # block); 2 and 4 rows per expert on
    # average (both forward GEMMs streaming, then down only); K of 4096 (the waves split
    # K; shorter K gives each wave its own column block), bf16 and NVFP4 activations
    compare_full(small("st_one", T=1, E=16, k=8))
    compare_full(small("st_2", T=8, E=16, k=4))
    compare_full(small("st_4", act_quant=True, H=768, I=384, T=16, E=16, k=4))
    compare_full(small("st_ks", H=256, I=4096, E=8, T=3, k=2))
    compare_full(small("st_ks_q", act_quant=True, H=256, I=4096, E=8, T=3, k=2))
    compare_full(small("st_zipf", logits="zipf", E=128, T=32, k=4), poison_empty=True)
    compare_full(small("st_skew", logits="skew", E=300, T=300, k=1, r=8))
    compare_full(small("st_odd", H=320, I=192, E=12, T=3, k=4))
    compare_full(small("st_w4a4", act_quant=True, H=768, I=384, E=16, T=4, k=4))
    compare_full(small("st_r72_sh", r=72, shared_a=True, E=32, T=8, k=4), lora_scale=0.5)
    compare_full(small("st_r0", r=0, E=16, T=4, k=4))
    compare_full(small("st_k64", H=64, I=64, E=8, T=2, k=2))


def test_fused_permutation_lora_a():
    # up to 16 tokens the permutation and the gate_up LoRA-A projection share one launch,
    # whose projection workgroups split K over 4, 2 or 1 waves per column as the grid
    # allows: 4 (T = 2), 2 (rank 72: a partial last column group) and 1 (T = 16, k = 8,
    # r = 64: 128 routed pairs; also with the shared A and NVFP4 activations)
    compare_full(small("fz_w4", T=2, E=16, k=4, r=64))
    compare_full(small("fz_w2", T=8, E=32, k=4, r=72), lora_scale=0.5)
    compare_full(small("fz_w1", T=16, E=32, k=8, r=64))
    compare_full(small("fz_w1_sh", T=16, E=32, k=8, r=64, shared_a=True, act_quant=True, H=768, I=384))


def test_decode_forward_graph_replay():
    # the decode-shaped forward (route + moe_fwd, the weight-streaming GEMMs) captured once
    # in a HIP graph and replayed: the library launches only kernels on the caller's stream
    # (no copies, fills or host synchronization), so every replay, with eager forwards on
    # other inputs and host synchronizations between the replays, gives the eager bits
    import torch
    import bit_quantized_moe_amd as bqm
    dev = gpu()
    shape = small("graph", T=4, E=16, k=4)
    ia = synth.layer_inputs(shape, device="cpu")
    ib = synth.layer_inputs(dataclasses.replace(shape, seed=shape.seed + 1), device="cpu")
    qgu = bqm.quantize_stack(ia.w_gu.to(dev), shape.fmt)
    qdn = bqm.quantize_stack(ia.w_dn.to(dev), shape.fmt)
    d = bqm.MoEDesc(shape.T, shape.H, shape.I, shape.E, shape.k, shape.r, qgu, qdn, A_gu=ia.A_gu.to(dev),
                    B_gu=ia.B_gu.to(dev), A_dn=ia.A_dn.to(dev), B_dn=ia.B_dn.to(dev))
    ws = torch.empty(bqm.bqm_moe_workspace_size(d), dtype=torch.uint8, device=dev)
    x = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=dev)
    lg = torch.empty((shape.T, shape.E), dtype=torch.float32, device=dev)
    idx = torch.empty((shape.T, shape.k), dtype=torch.int32, device=dev)
    tw = torch.empty((shape.T, shape.k), dtype=torch.float32, device=dev)
    out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=dev)

    def load(inp):
        x.copy_(inp.x.to(dev))
        lg.copy_(inp.logits.to(dev))

    def run():
        bqm.bqm_route(lg, shape.T, shape.E, shape.k, 0, idx, tw)
        bqm.bqm_moe_fwd(d, x, idx, tw, out, ws)

    ref = {}
    for name, inp in (("a", ia), ("b", ib)):
        load(inp)
        run()
        torch.cuda.synchronize()
        ref[name] = (out.clone(), idx.clone())
    assert not torch.equal(ref["a"][0], ref["b"][0])
    load(ia)
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
    for rep, name in enumerate("abab"):
        load(ia if name == "a" else ib)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[name][0]) and torch.equal(idx, ref[name][1]), f"replay {rep} ({name})"
        # eager work between the replays: a forward on the other input into other buffers
        other = ib if name == "a" else ia
        o2 = torch.empty_like(out)
        bqm.bqm_moe_fwd(d, other.x.to(dev), idx.clone(), tw.clone(), o2, ws)
        torch.cuda.synchronize()
    log("  graph replays match the eager forward bit for bit")


def test_few_rows_activation_dynamic_range():
    # a decode-sized batch (the 64-row tile configuration) whose tokens are scaled by
    # 2^40 and 2^-40, one all-zero token and one token whose elements span 2^-30 .. 2^30,
    # compared row by row (the whole-array norms would only see the largest row)
    import torch
    dev = gpu()
    shape = small("dec_range", T=24, E=16, k=4, r=16)
    inp = synth.layer_inputs(shape, device="cpu")
    x = inp.x.float()
    x[0] *= 2.0 ** 40
    x[1] *= 2.0 ** -40
    x[2] = 0.0
    x[3] *= torch.exp2(torch.linspace(-30.0, 30.0, shape.H).round())
    inp.x = x.to(torch.bfloat16)   # power-of-two factors: exact in bf16
    log(f"layer {shape} with rows scaled by 2^40, 2^-40, 0 and 2^-30..2^30")
    g = gpu_layer(inp, dev)
    o = oracle_layer(HostInputs(inp))
    assert (g["idx"].cpu().numpy() == o["idx"]).all(), "routing indices"
    out, dx = np_f32(g["out"]), np_f32(g["dx"])
    assert (out[2] == 0).all(), "an all-zero token gives an all-zero output"
    for t in range(shape.T):
        if t != 2:
            assert_close(out[t], o["out"][t], f"out row {t}")
        assert_close(dx[t], o["dx"][t], f"dx row {t}")
    assert_close(g["dtw"].cpu().numpy(), o["dtw"], "dtopk_w")
    for name, ref in zip(("dA_gu", "dB_gu", "dA_dn", "dB_dn"), o["lora"]):
        assert_close(g[name].cpu().numpy(), ref, name)


def test_tiny_workload():
    compare_full(synth.TINY)


def test_single_token_and_empty_batch():
    compare_full(small("one", T=1, k=4, E=8))
    import torch
    import bit_quantized_moe_amd as bqm
    dev = gpu()
    shape = small("empty", T=0)
    inp = synth.layer_inputs(dataclasses.replace(shape, T=1), device="cpu")
    g = gpu_layer(inp, dev)            # builds the weights; then call with T = 0
    d = g["desc"]
    d.T = 0
    ws = torch.empty(max(bqm.bqm_moe_workspace_size(d), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((1, shape.H), dtype=torch.bfloat16, device=dev)
    bqm.bqm_moe_fwd(d, None, None, None, None, ws)
    bqm.bqm_moe_dgrad(d, None, ws, None, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("shared_a", [False, True])
def test_deterministic_bitwise(shared_a):
    import torch
    dev = gpu()
    shape = small("det", T=150 if not shared_a else 1100, shared_a=shared_a)
    inp = synth.layer_inputs(shape, device="cpu")
    a = gpu_layer(inp, dev)
    b = gpu_layer(inp, dev)
    for k in ("out", "dx", "dtw", "dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype == torch.bfloat16 else b[k]), k


# ----------------------------------------------------------------------------
# full workload sizes: the GPU runs everything, the oracle checks sampled tokens
# (their output and input-gradient rows) and the LoRA gradients of sampled experts
# ----------------------------------------------------------------------------
def sampled_full(shape, tokens, lora_experts):
    import torch
    dev = gpu()
    log(f"full-size {shape.name}: generating inputs on the device")
    inp = synth.layer_inputs(shape, device=dev)
    g = gpu_layer(inp, dev)
    if lora_experts == "first":
        lora_experts = [int(g["idx"][tokens[0], 0])]
    log(f"  GPU layer done; oracle on tokens {tokens} and experts {lora_experts}")
    h = HostInputs(inp)
    o = oracle_layer(h, tokens=tokens, lora_experts=lora_experts)
    assert (g["idx"].cpu().numpy() == o["idx"]).all(), "routing indices"
    toks = o["tokens"]
    n_alt = resolve_w4a4_alternatives(np_f32(g["out"][toks]), None, o, h)
    log(f"  w4a4 rows with a valid alternative: {n_alt}")
    assert_close(np_f32(g["out"][toks]), o["out"], "out rows")
    assert_close(np_f32(g["dx"][toks]), o["dx"], "dx rows")
    assert_close(g["dtw"].cpu().numpy()[toks], o["dtw"][toks], "dtopk_w rows")
    for name, ref in zip(("dA_gu", "dB_gu", "dA_dn", "dB_dn"), o["lora"]):
        for e in lora_experts:
            assert_close(g[name][e].cpu().numpy(), ref[e], f"{name}[{e}]")
    # properties over the whole output: finite, and rows of tokens are not all zero
    assert torch.isfinite(g["out"].float()).all() and torch.isfinite(g["dx"].float()).all()
    log("  sampled parity ok")
    del g, inp
    torch.cuda.empty_cache()


def test_full_glm_sampled():
    sampled_full(synth.GLM, tokens=[0, 12345], lora_experts=[3])


def test_full_qwen_w4a4_sampled():
    # W4A4 quantizes a = silu(g) u per token after a GEMM: last-bit differences in
    # g, u (FP32 accumulation here, float64 in the oracle) move about 6e-4 of the
    # bf16 values of a to the other rounding neighbour; rows where that decides the
    # per-token scale are checked against the oracle's alternative (see
    # resolve_w4a4_alternatives).  24 tokens (192 routed rows) are sampled.
    toks = list(range(0, 8192, 8192 // 24))[:24]
    sampled_full(synth.QWEN, tokens=toks, lora_experts=[100])


def test_full_glm_decode_batch_sampled():
    # the GLM shape at T = 64 (about two rows per hit expert), as the decode-shaped
    # forward is timed: two tokens' rows and the LoRA gradients of token 0's first expert
    shape = dataclasses.replace(synth.GLM, T=64, name="glm_t64")
    sampled_full(shape, tokens=[0, 41], lora_experts="first")


def test_full_glm_streaming_forward_sampled():
    # the GLM shape at T = 32 (256 routed rows over 256 experts: the weight-streaming
    # forward), two tokens' rows and the LoRA gradients of token 0's first expert
    shape = dataclasses.replace(synth.GLM, T=32, name="glm_t32")
    sampled_full(shape, tokens=[0, 17], lora_experts="first")


def test_full_glm_nf4_sampled():
    sampled_full(synth.GLM_NF4, tokens=[1, 9000], lora_experts=[0])


def test_full_glm_nf4_nested_sampled():
    sampled_full(dataclasses.replace(synth.GLM_NF4, fmt="nf4_nested", name="glm_nf4_nested"),
                 tokens=[2, 7000], lora_experts=[5])


def test_full_glm_shared_lora_a_matches_replicated():
    # At the full GLM size the shared-A gradient sums all 131072 routed rows, more
    # than the oracle can take here.  Properties that hold at any size: the layer
    # with one shared A gives bit-identical out, dX and routing-weight gradients to
    # the per-expert layout holding E copies of that A (the kernels read the same
    # values), the B gradients are bit-identical, and the shared dA equals the sum of
    # the per-expert dA (the same per-expert FP32 sums, added in another order:
    # relative 1e-5).  Out and dX rows of two tokens are also checked against the
    # oracle.
    import torch
    dev = gpu()
    shape = dataclasses.replace(synth.GLM, name="glm_shared_a", shared_a=True)
    log("full-size GLM layer with a shared LoRA-A: generating inputs on the device")
    inp = synth.layer_inputs(shape, device=dev)
    sh = gpu_layer(inp, dev)
    rep_inp = dataclasses.replace(inp, shape=synth.GLM,
                                  A_gu=inp.A_gu.unsqueeze(0).expand(shape.E, -1, -1).contiguous(),
                                  A_dn=inp.A_dn.unsqueeze(0).expand(shape.E, -1, -1).contiguous())
    rep = gpu_layer(rep_inp, dev)
    for k in ("out", "dx", "dtw", "dB_gu", "dB_dn"):
        assert torch.equal(sh[k].view(torch.uint8) if sh[k].dtype == torch.bfloat16 else sh[k],
                           rep[k].view(torch.uint8) if rep[k].dtype == torch.bfloat16 else rep[k]), k
    for k in ("dA_gu", "dA_dn"):
        ref = rep[k].double().sum(0)
        err = (sh[k].double() - ref).norm() / ref.norm()
        log(f"  {k}: shared vs sum of per-expert, rel Frobenius {err.item():.2e}")
        assert err.item() < 1e-5, k
    del rep, rep_inp
    torch.cuda.empty_cache()
    h = HostInputs(inp)
    o = oracle_layer(h, tokens=[7, 15000])
    toks = o["tokens"]
    assert_close(np_f32(sh["out"][toks]), o["out"], "out rows")
    assert_close(np_f32(sh["dx"][toks]), o["dx"], "dx rows")
    log("  shared-A full-size checks ok")


# ----------------------------------------------------------------------------
# experts with several full 256-row tiles, every row compared
# ----------------------------------------------------------------------------
def big_experts(name, **kw):
    # R = 6000 routed rows over 8 experts; expert 0 gets the first 23% of the tokens on
    # top of its share (about 1270 rows: five row tiles, the last one ragged), the
    # others about 675 rows each (three row tiles)
    base = dict(E=8, H=1024, I=512, k=2, T=3000, r=16, seed=21, logits="skew")
    base.update(kw)
    return synth.Shape(name, **base)


def _check_rows_per_expert(o, E, least, most):
    counts = np.bincount(o["idx"].reshape(-1), minlength=E)
    log(f"  rows per expert {counts.tolist()}")
    assert counts.min() >= least and counts.max() >= most


def test_big_experts_nvfp4_every_row():
    g, o = compare_full(big_experts("big"), lora_scale=0.5)
    _check_rows_per_expert(o, 8, 600, 900)


def test_big_experts_w4a4_every_row():
    g, o = compare_full(big_experts("big_w4a4", act_quant=True))
    _check_rows_per_expert(o, 8, 600, 900)


def test_remainder_tiles():
    # about 525 rows per expert: an expert whose rows past its last full 256-row tile number
    # at most 64 has them computed by the 64-row kernels after the 256-row ones (forward, and
    # the NVFP4 dgrad; the others keep a partial 256-row tile); every row compared, NVFP4,
    # W4A4 and NF4 weights
    g, o = compare_full(small("rem", E=8, k=2, T=2100, r=16))
    counts = np.bincount(o["idx"].reshape(-1), minlength=8)
    rem = counts % 256
    assert ((rem > 0) & (rem <= 64)).any() and (rem > 64).any(), counts
    compare_full(small("rem_w4a4", E=8, k=2, T=2100, r=16, act_quant=True))
    compare_full(small("rem_nf4", E=8, k=2, T=2100, r=16, fmt="nf4"))


def test_lora_gradients_over_row_chunks():
    # the per-expert LoRA gradients cut an expert's rows into chunks of 2048 (one
    # workgroup per chunk, partial sums added in chunk order): with k = 1 over 3 experts
    # and 23% of the tokens pushed to expert 0, it gets about 3400 rows (two chunks), the
    # others about 1800 (one); every row of the layer compared
    g, o = compare_full(small("wgrad_chunks", E=3, k=1, T=7000, logits="skew", r=16))
    counts = np.bincount(o["idx"].reshape(-1), minlength=3)
    assert counts.max() > 2048 and counts.min() <= 2048, counts


def test_big_experts_nf4_every_row():
    g, o = compare_full(big_experts("big_nf4", fmt="nf4"))
    _check_rows_per_expert(o, 8, 600, 900)


def test_lora_rank_72_and_128():
    # r = 72: the LoRA projections' partial 64-column tile and the masked K tail of the
    # up-projection segment; r = 128: two projection column tiles, U/V rows of 256
    compare_full(small("r72", r=72), lora_scale=0.5)
    compare_full(small("r128", r=128, H=320, I=192, T=260, E=12))
    compare_full(small("r72_sh", r=72, shared_a=True, T=400))
    compare_full(small("r128_nf4", r=128, fmt="nf4", logits="zipf", E=32, T=200), poison_empty=True)


@pytest.mark.parametrize("T,bad", [(120, [(3, 1, -1), (50, 0, 16), (50, 3, 1000), (119, 2, -7)]),
                                   (12, [(3, 1, -1), (5, 0, 16), (5, 3, 1000), (11, 2, -7)])])
def test_out_of_range_expert_indices_are_dropped(T, bad):
    # caller-supplied indices outside [0, E) belong to no expert: the permutation puts
    # those pairs after offsets[E], and they add nothing to out, dX or the LoRA
    # gradients (their routing-weight gradient is 0).  The oracle sees the same layer
    # with those pairs' routing weights set to 0 (any expert stands in for them).
    # T = 120 sorts in three passes; T = 12 runs the one-workgroup permutation fused
    # with the gate_up LoRA-A projection, whose workgroups skip the dropped pairs
    import torch
    import bit_quantized_moe_amd as bqm
    dev = gpu()
    shape = small("dropped", T=T, E=16, k=4, r=8)
    inp = synth.layer_inputs(shape, device="cpu")
    h = HostInputs(inp)
    idx, tw = __import__("oracle.routing", fromlist=["route"]).route(h.logits, shape.k)
    idx = idx.copy()
    tw = tw.copy()
    for t, j, v in bad:
        idx[t, j] = v
    # oracle: the dropped pairs go to an expert the token does not use, with weight 0
    idx_o = idx.copy()
    for t, j, _ in bad:
        idx_o[t, j] = next(e for e in range(shape.E) if e not in idx[t])
        tw[t, j] = 0.0
    w = h.weights()
    from oracle import moe as om
    out_o, cache = om.forward(w, h.x, idx_o, tw)
    dx_o, dtw_o, bwd = om.dgrad(w, cache, h.dout, tw)
    lora_o = om.lora_grad(w, cache, bwd, shape.E)

    x, dout = inp.x.to(dev), inp.dout.to(dev)
    qgu = bqm.quantize_stack(inp.w_gu.to(dev), "nvfp4")
    qdn = bqm.quantize_stack(inp.w_dn.to(dev), "nvfp4")
    idx_g = torch.from_numpy(idx.astype(np.int32)).to(dev)
    tw_g = torch.from_numpy(tw.astype(np.float32)).to(dev)
    # the permutation alone: offsets[E] counts the pairs that have an expert
    R = shape.T * shape.k
    perm = torch.empty(R, dtype=torch.int32, device=dev)
    inv = torch.empty(R, dtype=torch.int32, device=dev)
    off = torch.empty(shape.E + 1, dtype=torch.int32, device=dev)
    pws = torch.empty(max(bqm.bqm_permute_workspace_size(shape.T, shape.E, shape.k), 16), dtype=torch.uint8,
                      device=dev)
    bqm.bqm_permute(idx_g, shape.T, shape.E, shape.k, perm, inv, off, pws)
    torch.cuda.synchronize()
    assert int(off[-1]) == R - len(bad)
    p = perm.cpu().numpy()
    assert sorted(p.tolist()) == list(range(R)) and (inv.cpu().numpy()[p] == np.arange(R)).all()
    assert sorted(p[R - len(bad):].tolist()) == sorted(t * shape.k + j for t, j, _ in bad)

    lor = dict(A_gu=inp.A_gu.to(dev), B_gu=inp.B_gu.to(dev), A_dn=inp.A_dn.to(dev), B_dn=inp.B_dn.to(dev))
    d = bqm.MoEDesc(shape.T, shape.H, shape.I, shape.E, shape.k, shape.r, qgu, qdn, **lor)
    ws = torch.empty(bqm.bqm_moe_workspace_size(d), dtype=torch.uint8, device=dev)
    out = torch.empty((shape.T, shape.H), dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(out)
    dtw = torch.empty((shape.T, shape.k), dtype=torch.float32, device=dev)
    bqm.bqm_moe_fwd(d, x, idx_g, tw_g, out, ws)
    bqm.bqm_moe_dgrad(d, dout, ws, dx, dtw)
    gr = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in lora_o]
    bqm.bqm_lora_grad(d, x, dout, ws, *gr)
    torch.cuda.synchronize()
    assert_close(np_f32(out), out_o, "out")
    assert_close(np_f32(dx), dx_o, "dx")
    keep = np.ones((shape.T, shape.k), bool)
    for t, j, _ in bad:
        keep[t, j] = False
    g_dtw = dtw.cpu().numpy()
    assert_close(g_dtw[keep], dtw_o[keep], "dtopk_w")
    assert (g_dtw[~keep] == 0).all()
    for name, got, ref in zip(("dA_gu", "dB_gu", "dA_dn", "dB_dn"), gr, lora_o):
        assert_close(got.cpu().numpy(), ref, name)
