"""Pins of the oracle's float64 MoE forward, dgrad and LoRA gradients.

Pinned against: explicit scalar loops of the definition, torch float64 autograd
of the same forward (weights held as constants), central finite differences,
and invariants (routed-only dequantization, W4A4 batch invariance).
"""
import numpy as np
import pytest
import torch

from oracle import formats as fm
from oracle import moe as om
from oracle import quant as oq
from oracle import routing as orr


def _bf16(a):
    return fm.bf16_round(np.asarray(a, dtype=np.float32))


def make_layer(E=4, H=32, I=16, k=2, T=6, r=4, seed=0, fmt="nvfp4", act_quant=False, s=1.0, shared_a=False):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)))
    wgu = _bf16(rng.standard_normal((E, 2 * I, H)) * 0.2)
    wdn = _bf16(rng.standard_normal((E, H, I)) * 0.2)
    A_gu = _bf16(rng.standard_normal((E, r, H)) * 0.1)
    B_gu = _bf16(rng.standard_normal((E, 2 * I, r)) * 0.1)
    A_dn = _bf16(rng.standard_normal((E, r, I)) * 0.1)
    B_dn = _bf16(rng.standard_normal((E, H, r)) * 0.1)
    if shared_a:
        A_gu, A_dn = A_gu[0], A_dn[0]
    if fmt == "nvfp4":
        gu, dn = oq.quantize_nvfp4(wgu), oq.quantize_nvfp4(wdn)
    else:
        gu, dn = oq.quantize_nf4(wgu), oq.quantize_nf4(wdn)
    w = om.MoEWeights(fmt, gu, dn, A_gu, B_gu, A_dn, B_dn, lora_scale=s, act_quant=act_quant,
                      shared_a=shared_a)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, tw = orr.route(lg, k)
    dout = _bf16(rng.standard_normal((T, H)))
    return w, x, idx, tw, dout, (wgu, wdn)


def _loops_forward(w, x, idx, tw, round_points=True):
    """The definition with scalar Python loops (float64), no matrix products."""
    T, H = x.shape
    k = idx.shape[1]
    s = w.lora_scale
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            Wgu = om.expert_matrix(w.gu, e)
            Wdn = om.expert_matrix(w.dn, e)
            I = Wdn.shape[1]
            r = w.A_gu.shape[1]
            xt = [float(v) for v in x[t]]
            U = [sum(float(w.A_gu[e, q, c]) * xt[c] for c in range(H)) for q in range(r)]
            h = []
            for n in range(2 * I):
                base = sum(Wgu[n, c] * xt[c] for c in range(H))
                lora = sum(float(w.B_gu[e, n, q]) * U[q] for q in range(r))
                h.append(base + s * lora)
            a = []
            for i in range(I):
                g, u = h[i], h[I + i]
                val = g / (1.0 + np.exp(-g)) * u
                a.append(float(_bf16([val])[0]) if round_points else val)
            Ud = [sum(float(w.A_dn[e, q, i]) * a[i] for i in range(I)) for q in range(r)]
            for c in range(H):
                y = sum(Wdn[c, i] * a[i] for i in range(I))
                y += s * sum(float(w.B_dn[e, c, q]) * Ud[q] for q in range(r))
                out[t, c] += tw[t, j] * y
    return out


def test_forward_matches_scalar_loops():
    w, x, idx, tw, _, _ = make_layer(E=3, H=16, I=16, k=2, T=4, r=2, seed=1, s=0.5)
    out, _ = om.forward(w, x, idx, tw)
    ref = _loops_forward(w, x, idx, tw)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def _torch_layer(w, x, idx, tw):
    """Same forward in torch float64 (pure chain, no rounding points) for autograd."""
    xs = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    tws = torch.tensor(np.asarray(tw, np.float64), requires_grad=True)
    lora = {n: torch.tensor(getattr(w, n).astype(np.float64), requires_grad=True)
            for n in ("A_gu", "B_gu", "A_dn", "B_dn")}
    T, H = x.shape
    k = idx.shape[1]
    s = w.lora_scale
    out = torch.zeros((T, H), dtype=torch.float64)
    for e in range(w.B_gu.shape[0]):
        tt, jj = np.nonzero(idx == e)
        if tt.size == 0:
            continue
        Wgu = torch.tensor(om.expert_matrix(w.gu, e))
        Wdn = torch.tensor(om.expert_matrix(w.dn, e))
        # a shared A is one leaf that every expert reads: autograd sums its uses
        Agu = lora["A_gu"] if w.shared_a else lora["A_gu"][e]
        Adn = lora["A_dn"] if w.shared_a else lora["A_dn"][e]
        X = xs[tt]
        h = X @ Wgu.T + s * (X @ Agu.T) @ lora["B_gu"][e].T
        I = Wdn.shape[1]
        g, u = h[:, :I], h[:, I:]
        a = torch.nn.functional.silu(g) * u
        y = a @ Wdn.T + s * (a @ Adn.T) @ lora["B_dn"][e].T
        out = out.index_add(0, torch.tensor(tt), y * tws[tt, jj][:, None])
    return out, xs, tws, lora


def test_dgrad_and_lora_grads_match_torch_autograd():
    w, x, idx, tw, dout, _ = make_layer(E=4, H=32, I=16, k=2, T=9, r=4, seed=2, s=0.7)
    out, cache = om.forward(w, x, idx, tw, round_points=False)
    dX, dtw, bwd = om.dgrad(w, cache, dout, tw, round_points=False)
    dA_gu, dB_gu, dA_dn, dB_dn = om.lora_grad(w, cache, bwd, E=4)
    tout, xs, tws, lora = _torch_layer(w, x, idx, tw)
    assert np.allclose(out, tout.detach().numpy(), rtol=1e-12, atol=1e-12)
    tout.backward(torch.tensor(np.asarray(dout, np.float64)))
    assert np.allclose(dX, xs.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dtw, tws.grad.numpy(), rtol=1e-10, atol=1e-12)
    for mine, name in ((dA_gu, "A_gu"), (dB_gu, "B_gu"), (dA_dn, "A_dn"), (dB_dn, "B_dn")):
        assert np.allclose(mine, lora[name].grad.numpy(), rtol=1e-10, atol=1e-12), name


def test_shared_a_grads_match_torch_autograd():
    # one LoRA-A for every expert (the GLM page's adapter layout): its gradient is
    # the sum of every expert's use; E=5 with T=7, k=2 leaves room for an idle expert
    w, x, idx, tw, dout, _ = make_layer(E=5, H=32, I=16, k=2, T=7, r=4, seed=12, s=0.6, shared_a=True)
    out, cache = om.forward(w, x, idx, tw, round_points=False)
    dX, dtw, bwd = om.dgrad(w, cache, dout, tw, round_points=False)
    dA_gu, dB_gu, dA_dn, dB_dn = om.lora_grad(w, cache, bwd, E=5)
    assert dA_gu.shape == w.A_gu.shape and dA_dn.shape == w.A_dn.shape
    tout, xs, tws, lora = _torch_layer(w, x, idx, tw)
    assert np.allclose(out, tout.detach().numpy(), rtol=1e-12, atol=1e-12)
    tout.backward(torch.tensor(np.asarray(dout, np.float64)))
    assert np.allclose(dX, xs.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dtw, tws.grad.numpy(), rtol=1e-10, atol=1e-12)
    for mine, name in ((dA_gu, "A_gu"), (dB_gu, "B_gu"), (dA_dn, "A_dn"), (dB_dn, "B_dn")):
        assert np.allclose(mine, lora[name].grad.numpy(), rtol=1e-10, atol=1e-12), name


def test_shared_a_central_finite_differences():
    # d<dOut, out>/dA along a random direction, for the shared gate_up and down A
    w, x, idx, tw, dout, _ = make_layer(E=3, H=16, I=16, k=2, T=5, r=2, seed=13, s=0.8, shared_a=True)
    x64 = np.asarray(x, np.float64)
    d64 = np.asarray(dout, np.float64)
    _, cache = om.forward(w, x64, idx, tw, round_points=False)
    _, _, bwd = om.dgrad(w, cache, d64, tw, round_points=False)
    grads = om.lora_grad(w, cache, bwd, E=3)
    rng = np.random.default_rng(1)
    eps = 1e-3
    for name, g in (("A_gu", grads[0]), ("A_dn", grads[2])):
        base = getattr(w, name).astype(np.float64)
        v = rng.standard_normal(base.shape)

        def loss(a):
            wv = om.MoEWeights(w.fmt, w.gu, w.dn, **{**dict(A_gu=w.A_gu, B_gu=w.B_gu, A_dn=w.A_dn, B_dn=w.B_dn),
                                                      name: a}, lora_scale=w.lora_scale, shared_a=True)
            return (om.forward(wv, x64, idx, tw, round_points=False)[0] * d64).sum()
        fd = (loss(base + eps * v) - loss(base - eps * v)) / (2 * eps)
        assert np.isclose(fd, (g * v).sum(), rtol=1e-6), name


def test_shared_a_equals_replicated_per_expert_a():
    # the shared layout is the per-expert layout with E equal slices: same outputs,
    # and the shared gradient is the sum of the per-expert ones (rounding points on)
    w, x, idx, tw, dout, _ = make_layer(E=4, H=32, I=16, k=2, T=9, r=4, seed=14, s=0.5, shared_a=True)
    rep = om.MoEWeights(w.fmt, w.gu, w.dn, np.repeat(w.A_gu[None], 4, 0), w.B_gu,
                        np.repeat(w.A_dn[None], 4, 0), w.B_dn, lora_scale=w.lora_scale)
    o1, c1 = om.forward(w, x, idx, tw)
    o2, c2 = om.forward(rep, x, idx, tw)
    assert (o1 == o2).all()
    d1, t1, b1 = om.dgrad(w, c1, dout, tw)
    d2, t2, b2 = om.dgrad(rep, c2, dout, tw)
    assert (d1 == d2).all() and (t1 == t2).all()
    g1 = om.lora_grad(w, c1, b1, E=4)
    g2 = om.lora_grad(rep, c2, b2, E=4)
    assert np.allclose(g1[0], g2[0].sum(0), rtol=1e-13, atol=1e-15)
    assert np.allclose(g1[2], g2[2].sum(0), rtol=1e-13, atol=1e-15)
    assert (g1[1] == g2[1]).all() and (g1[3] == g2[3]).all()


def test_dgrad_central_finite_differences():
    w, x, idx, tw, dout, _ = make_layer(E=3, H=16, I=16, k=2, T=5, r=2, seed=3)
    x64 = np.asarray(x, np.float64)
    d64 = np.asarray(dout, np.float64)
    _, cache = om.forward(w, x64, idx, tw, round_points=False)
    dX, dtw, _ = om.dgrad(w, cache, d64, tw, round_points=False)
    rng = np.random.default_rng(0)
    v = rng.standard_normal(x64.shape)
    eps = 1e-3
    fp = (om.forward(w, x64 + eps * v, idx, tw, round_points=False)[0] * d64).sum()
    fm_ = (om.forward(w, x64 - eps * v, idx, tw, round_points=False)[0] * d64).sum()
    fd = (fp - fm_) / (2 * eps)
    assert np.isclose(fd, (dX * v).sum(), rtol=1e-6)
    vw = rng.standard_normal(tw.shape)
    fp = (om.forward(w, x64, idx, tw + eps * vw, round_points=False)[0] * d64).sum()
    fm_ = (om.forward(w, x64, idx, tw - eps * vw, round_points=False)[0] * d64).sum()
    assert np.isclose((fp - fm_) / (2 * eps), (dtw * vw).sum(), rtol=1e-8)


def test_rounding_points_are_small_perturbations():
    w, x, idx, tw, dout, _ = make_layer(E=4, H=64, I=32, k=2, T=16, r=4, seed=4)
    o1, c1 = om.forward(w, x, idx, tw, round_points=True)
    o0, c0 = om.forward(w, x, idx, tw, round_points=False)
    fro, _ = om.rel_errors(o1, o0)
    assert 0 < fro < 5e-3
    d1, _, _ = om.dgrad(w, c1, dout, tw, round_points=True)
    d0, _, _ = om.dgrad(w, c0, dout, tw, round_points=False)
    fro, _ = om.rel_errors(d1, d0)
    assert 0 < fro < 5e-3


def test_token_subset_rows_equal_full_rows():
    for aq in (False, True):
        w, x, idx, tw, dout, _ = make_layer(E=4, H=32, I=16, k=2, T=12, r=4, seed=5, act_quant=aq)
        full, cf = om.forward(w, x, idx, tw)
        sub, cs = om.forward(w, x, idx, tw, tokens=[2, 7, 11])
        # equal up to float64 summation order inside the matrix products
        assert np.allclose(sub, full[[2, 7, 11]], rtol=1e-12, atol=1e-14)
        dfull, _, _ = om.dgrad(w, cf, dout, tw)
        dsub, _, _ = om.dgrad(w, cs, dout, tw)
        assert np.allclose(dsub, dfull[[2, 7, 11]], rtol=1e-12, atol=1e-14)


def test_w4a4_uses_quantized_activations_and_differs_from_w4a16():
    w, x, idx, tw, _, _ = make_layer(E=4, H=64, I=32, k=2, T=10, r=4, seed=6, act_quant=True)
    out_q, _ = om.forward(w, x, idx, tw)
    w.act_quant = False
    out_b, _ = om.forward(w, x, idx, tw)
    fro, _ = om.rel_errors(out_q, out_b)
    assert 0.01 < fro < 0.3


def test_routed_only_dequantization():
    """Experts that get no token are never read: poisoning their scales changes nothing."""
    w, x, idx, tw, dout, _ = make_layer(E=6, H=32, I=16, k=2, T=5, r=4, seed=7)
    idx = np.where(idx >= 4, idx % 4, idx)           # experts 4, 5 get no token
    idx[:, 1] = np.where(idx[:, 1] == idx[:, 0], (idx[:, 0] + 1) % 4, idx[:, 1])
    out, c = om.forward(w, x, idx, tw)
    dX, dtw, _ = om.dgrad(w, c, dout, tw)
    w.gu.scales[4:] = 0x7F                           # E4M3 NaN
    w.dn.scales[4:] = 0x7F
    out2, c2 = om.forward(w, x, idx, tw)
    dX2, dtw2, b2 = om.dgrad(w, c2, dout, tw)
    assert np.isfinite(out2).all() and (out2 == out).all() and (dX2 == dX).all()
    grads = om.lora_grad(w, c2, b2, E=6)
    for g in grads:
        assert (g[4:] == 0).all()


def test_nf4_against_bf16_sanity_band():
    """NF4 vs unquantized weights: output error of the order the nf4moe page reports (0.15)."""
    w, x, idx, tw, dout, (wgu, wdn) = make_layer(E=4, H=128, I=64, k=2, T=32, r=4, seed=8, fmt="nf4")
    out_q, cq = om.forward(w, x, idx, tw)
    dq, _, _ = om.dgrad(w, cq, dout, tw)
    ref = om.MoEWeights("nvfp4", None, None, w.A_gu, w.B_gu, w.A_dn, w.B_dn)
    saved = om.expert_matrix
    try:
        om.expert_matrix = lambda q, e: (wgu if q == "gu" else wdn)[e].astype(np.float64)
        ref.gu, ref.dn = "gu", "dn"
        out_b, cb = om.forward(ref, x, idx, tw)
        db, _, _ = om.dgrad(ref, cb, dout, tw)
    finally:
        om.expert_matrix = saved
    fro, _ = om.rel_errors(out_q, out_b)
    cos = (dq * db).sum() / np.linalg.norm(dq) / np.linalg.norm(db)
    assert 0.03 < fro < 0.3
    assert cos > 0.97


def test_nf4_nested_layer_is_the_layer_over_its_dequantized_weights():
    # the nested-absmax NF4 layer equals the plain-NF4 layer whose absmax is replaced
    # by absmax' (the forward and dgrad see only the dequantized weights), and it
    # stays close to the plain NF4 layer (absmax' within 2^-4 of each group's max |d|)
    w, x, idx, tw, dout, (wgu, wdn) = make_layer(E=4, H=128, I=64, k=2, T=9, r=4, seed=15, fmt="nf4")
    ngu, ndn = oq.nest_absmax(w.gu), oq.nest_absmax(w.dn)
    wn = om.MoEWeights("nf4", ngu, ndn, w.A_gu, w.B_gu, w.A_dn, w.B_dn)
    wp = om.MoEWeights("nf4", oq.NF4Tensor(ngu.codes, oq.unnest_absmax(ngu)),
                       oq.NF4Tensor(ndn.codes, oq.unnest_absmax(ndn)), w.A_gu, w.B_gu, w.A_dn, w.B_dn)
    o1, c1 = om.forward(wn, x, idx, tw)
    o2, c2 = om.forward(wp, x, idx, tw)
    assert (o1 == o2).all()
    assert (om.dgrad(wn, c1, dout, tw)[0] == om.dgrad(wp, c2, dout, tw)[0]).all()
    o3, _ = om.forward(w, x, idx, tw)
    assert 0 < np.linalg.norm(o1 - o3) / np.linalg.norm(o3) < 0.05


def test_w4a4_operand_split_hand_derived():
    """W4A4 on one token and one expert, every value derived by hand (4-bitter page,
    section "Method": per-token NVFP4 activations feed the base GEMMs, the LoRA path
    stays bf16; the backward keeps bf16 operands, so the quantizers pass gradients
    through).  The pin fails if LoRA reads DQ(Q(X)) instead of X, if a is quantized
    before its bf16 rounding, if the down LoRA reads DQ(Q(a_b)), or if the dgrad's
    SwiGLU derivative uses the unquantized forward.

    X = [4, 5, 6, 0, ..., 0] is row 1 of the GLM page's worked example padded to one
    16-block.  Per token, amax = 6 gives s_dec = 6 / (6 * 256) = 2^-8, so the scaled
    row is y = [1024, 1280, 1536] (t = 1536).  Scale-to-6: sb = 256, y / sb = [4, 5, 6],
    5 ties between 4 and 6 and goes to the even code (4), error 256^2 = 65536.
    Scale-to-4: sb = 384, y / sb = [2.67, 3.33, 4] -> [3, 3, 4], q * sb = [1152, 1152,
    1536], error 128^2 + 128^2 = 32768 < 65536, so 4 wins: DQ(Q_row(X)) = [4.5, 4.5, 6].
    The weights hold 0, 1 and one 6 that meets only zeros: amax 6 gives s_dec = 2^-8
    exactly, and a block holding a single 1 scales to t = 256, where scale-to-4 (sb =
    64, code 4: 256) is exact and beats scale-to-6 (sb = e4m3(42.7) = 44, code 6: 264),
    so DQ = 1 exactly.  A row of a with a single nonzero v: t = fl(v * fl(1 / fl(v / 1536)))
    lies within a few ulps of 1536, so both candidates give q * sb = 1536 (6 * 256 and
    4 * 384; the tie keeps 6) and DQ = 1536 * fl32(v / 1536)."""
    H = I = 16
    x = np.zeros((1, H), np.float32)
    x[0, :3] = [4, 5, 6]
    wgu = np.zeros((1, 2 * I, H), np.float32)
    wgu[0, 0, 0] = 1.0        # gate 0 reads x0
    wgu[0, I, 2] = 1.0        # up 0 reads x2
    wgu[0, 2 * I - 1, H - 1] = 6.0   # up 15 reads x15 = 0
    wdn = np.zeros((1, H, I), np.float32)
    wdn[0, 0, 0] = 1.0        # y0 reads a0
    wdn[0, H - 1, I - 1] = 6.0       # y15 reads a15 = 0
    A_gu = np.zeros((1, 1, H), np.float32)
    A_gu[0, 0, 0] = 1.0       # U_gu = x0
    B_gu = np.zeros((1, 2 * I, 1), np.float32)
    B_gu[0, 0, 0] = 0.25      # gate 0 += 0.25 U_gu
    A_dn = np.zeros((1, 1, I), np.float32)
    A_dn[0, 0, 0] = 1.0       # U_dn = a0
    B_dn = np.zeros((1, H, 1), np.float32)
    B_dn[0, 0, 0] = 0.5       # y0 += 0.5 U_dn
    B_dn[0, 5, 0] = 0.25      # y5 = 0.25 U_dn (LoRA only)
    w = om.MoEWeights("nvfp4", oq.quantize_nvfp4(wgu), oq.quantize_nvfp4(wdn), A_gu, B_gu, A_dn, B_dn,
                      act_quant=True)
    assert (om.expert_matrix(w.gu, 0) == wgu[0]).all() and (om.expert_matrix(w.dn, 0) == wdn[0]).all()
    assert (om.act_dq(x) == np.array([[4.5, 4.5, 6] + [0] * 13])).all()
    idx = np.zeros((1, 1), np.int32)
    tw = np.ones((1, 1))
    out, cache = om.forward(w, x, idx, tw)

    def silu(v):
        return v / (1.0 + np.exp(-v))

    g0 = 4.5 + 0.25 * 4.0                 # base on DQ(Q_row(X))[0], LoRA on the bf16 x0
    u0 = 6.0                              # DQ(Q_row(X))[2]
    a_b0 = float(torch.tensor(silu(g0) * u0, dtype=torch.float64).to(torch.bfloat16).double())
    dq_a0 = 1536.0 * float(np.float32(a_b0) / np.float32(1536.0))
    want = np.zeros(H)
    want[0] = dq_a0 + 0.5 * a_b0
    want[5] = 0.25 * a_b0
    assert np.allclose(out[0], want, rtol=1e-14, atol=0)

    # each misreading moves the result far outside that tolerance
    g_bad = 4.5 + 0.25 * 4.5              # LoRA on DQ(Q(X))
    a_bad = float(torch.tensor(silu(g_bad) * u0, dtype=torch.float64).to(torch.bfloat16).double())
    unrounded = silu(g0) * u0             # a quantized before its bf16 rounding
    dq_unrounded = 1536.0 * float(np.float32(unrounded) / np.float32(1536.0))
    for alt in (dq_unrounded + 0.5 * unrounded, 1536.0 * float(np.float32(a_bad) / np.float32(1536.0)) + 0.5 * a_bad,
                dq_a0 + 0.5 * dq_a0):     # the last: down LoRA on DQ(Q(a_b))
        assert abs(alt - want[0]) > 1e-9 * abs(want[0])

    # dgrad with dOut = e0 + e5: da_u0 = 1 (W_dn) + (1 * 0.5 + 1 * 0.25) * 1 (LoRA) = 1.75;
    # SwiGLU' at the forward's g0 = 5.5 and u0 = 6; dX0 = dg (W_gu) + 0.25 dg (LoRA), dX2 = du
    dout = np.zeros((1, H), np.float32)
    dout[0, 0] = dout[0, 5] = 1.0
    dX, dtw, _ = om.dgrad(w, cache, dout, tw)
    sg = 1.0 / (1.0 + np.exp(-g0))
    dg = float(torch.tensor(1.75 * u0 * sg * (1 + g0 * (1 - sg)), dtype=torch.float64).to(torch.bfloat16).double())
    du = float(torch.tensor(1.75 * silu(g0), dtype=torch.float64).to(torch.bfloat16).double())
    want_dx = np.zeros(H)
    want_dx[0] = dg + 0.25 * dg
    want_dx[2] = du
    assert np.allclose(dX[0], want_dx, rtol=1e-14, atol=0)
    assert np.isclose(dtw[0, 0], want[0] + want[5], rtol=1e-14)
    g_st = 4.0 + 0.25 * 4.0               # SwiGLU' at the unquantized forward instead
    sgb = 1.0 / (1.0 + np.exp(-g_st))
    assert abs(1.75 * 4.0 * sgb * (1 + g_st * (1 - sgb)) * 1.25 - want_dx[0]) > 1e-3
