"""Pins of the oracle's expert GEMMs, SwiGLU, requant and finalize.

The weights are decoded here independently of the oracle's tables (E2M1 from
the OCP value list typed below, E4M3 through torch's float8_e4m3fn, E8M0 as
2^(c-127)) and the layer is recomposed with numpy matmuls in fp64:
  * E = k = 1, scale 1, no shared expert reduces to the textbook SwiGLU MLP
    followed by the residual add and RMSNorm;
  * k = E is the dense mixture; k < E equals the dense sum with zero weight on
    the experts a row did not choose;
  * bumping every W2 scale code by one (MX) or doubling every W2 global (NV)
    doubles every expert output exactly;
  * the finalize reduces to textbook RMSNorm when the experts contribute 0,
    and to sign(v)*gamma on a constant row.
The quantization steps inside the layer are the oracle's own encoders, which
are pinned by exhaustive searches in test_oracle_formats.py.
"""
import numpy as np
import pytest
import torch

from block_scaled_fp4_sigmoid_amd import synth

# OCP MX v1.0 FP4 (E2M1) values for codes 0..15.
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


def bf16v(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3v(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dense(m: synth.Matrix) -> np.ndarray:
    """Independent decode of a synthetic weight matrix to fp64 [N, K]."""
    if m.fmt == synth.BF16:
        return bf16v(m.bf16)
    lo = m.packed & 15
    hi = m.packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(m.N, m.K)
    v = E2M1[codes]
    if m.fmt == synth.MXFP4:
        sc = np.exp2(m.scales.astype(np.float64) - 127)
        return v * np.repeat(sc, 32, axis=1)
    sc = e4m3v(m.scales) * np.float64(np.float32(m.gscale))
    return v * np.repeat(sc, 16, axis=1)


def mx_dequant(q, s):
    return e4m3v(q) * np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=-1)


def clamp_gu(g, u, limit):
    """The clamped SwiGLU's inputs: gate capped from above, up clamped both ways."""
    if limit > 0:
        g, u = np.minimum(g, limit), np.clip(u, -limit, limit)
    return g, u


def textbook_expert(orc, m13, m2, I, a, limit=0.0, h_g=None):
    """a: dequantized activation [H]; returns y [H] with the layer's requant of
    h: MXFP8, or NVFP4 with global h_g (the rule reads h in fp32)."""
    W13, W2 = dense(m13), dense(m2)
    g, u = clamp_gu(W13[:I] @ a, W13[I:] @ a, limit)
    h = g / (1 + np.exp(-g)) * u
    if h_g is not None:
        q, s = orc.nvfp4_quant_f32(h[None, :].astype(np.float32), h_g)
        return W2 @ orc.nvfp4_dequant(q, s, h_g)[0]
    q, s = orc.mxfp8_quant_f64(h[None, :])
    return W2 @ mx_dequant(q, s)[0]


def textbook_norm(orc, t, gamma, eps):
    rb = orc.bf16_rne_n(t).astype(np.uint16)
    r = bf16v(rb)
    return r / np.sqrt(np.mean(r * r) + eps) * bf16v(gamma), rb


def _layer(orc, shape, seed, **kw):
    inp = synth.make_inputs(shape, seed=seed, pool_rows=kw.get("pool_rows", 4096))
    return inp, orc.Layer(inp)


def _act(orc, inp, r):
    if inp.shape.act_fmt == synth.ACT_NVFP4:
        q, s = orc.nvfp4_quant_bf16(inp.x[r:r + 1], inp.x_gscale)
        return orc.nvfp4_dequant(q, s, inp.x_gscale)[0]
    q, s = orc.mxfp8_quant_bf16(inp.x[r:r + 1])
    return mx_dequant(q, s)[0]


@pytest.mark.parametrize("wfmt", [synth.MXFP4, synth.NVFP4])
def test_single_expert_is_textbook_swiglu_mlp(orc, wfmt):
    sh = synth.custom_shape(M=3, H=256, E=1, k=1, I=64, wfmt=wfmt, routed_scale=1.0)
    inp, L = _layer(orc, sh, 5)
    res = L.rows(np.arange(3))
    for r in range(3):
        a = _act(orc, inp, r)
        y = textbook_expert(orc, inp.w13.expert(0), inp.w2.expert(0), sh.I, a)
        out, rb = textbook_norm(orc, bf16v(inp.x[r]) + y, inp.gamma, sh.eps)
        assert res["ids"][r, 0] == 0 and res["w"][r, 0] == 1.0
        assert np.allclose(res["y"][r, 0], y, rtol=1e-12, atol=1e-15)
        assert np.array_equal(res["resid_out"][r], rb)
        assert np.allclose(res["out64"][r], out, rtol=1e-12, atol=1e-14)


A4 = synth.ACT_NVFP4


@pytest.mark.parametrize("wfmt,sfmt,limit,act", [(synth.MXFP4, synth.NONE, 0.0, 0), (synth.NVFP4, synth.BF16, 0.0, 0),
                                                 (synth.MXFP4, synth.MXFP4, 0.0, 0), (synth.NVFP4, synth.BF16, 0.06, 0),
                                                 (synth.MXFP4, synth.MXFP4, 0.05, 0), (synth.NVFP4, synth.NONE, 0.0, A4),
                                                 (synth.NVFP4, synth.NVFP4, 0.0, A4), (synth.NVFP4, synth.BF16, 0.06, A4)])
def test_sparse_routing_equals_dense_zero_weighted_mixture(orc, wfmt, sfmt, limit, act):
    """Also with the clamped SwiGLU (limit > 0, small enough that most gate and
    up values of these rows cross it) in the routed and the shared experts, and
    with NVFP4 activations (the input and each h quantized with their globals)."""
    sh = synth.custom_shape(M=4, H=128, E=6, k=3, I=64, wfmt=wfmt, sfmt=sfmt, I_sh=96,
                            routed_scale=2.5, bias="normal:0.05", swiglu_limit=limit, act_fmt=act)
    inp, L = _layer(orc, sh, 6)
    inp = synth.vary_globals(inp, 9)
    L = orc.Layer(inp)
    res = L.rows(np.arange(sh.M))
    for r in range(sh.M):
        a = _act(orc, inp, r)
        hg = (lambda e: float(inp.h_gscale[e])) if act == A4 else (lambda e: None)
        ys = np.stack([textbook_expert(orc, inp.w13.expert(e), inp.w2.expert(e), sh.I, a, limit, hg(e))
                       for e in range(sh.E)])
        wd = np.zeros(sh.E)
        wd[res["ids"][r]] = res["w"][r]  # zero weight on unchosen experts
        t = bf16v(inp.x[r]) + wd @ ys
        if sfmt == synth.BF16:
            W13, W2 = dense(inp.sh13), dense(inp.sh2)
            xv = bf16v(inp.x[r])
            g, u = clamp_gu(W13[:sh.I_sh] @ xv, W13[sh.I_sh:] @ xv, limit)
            hb = bf16v(orc.bf16_rne_n(g / (1 + np.exp(-g)) * u))
            t = t + W2 @ hb
        elif sfmt in (synth.MXFP4, synth.NVFP4):
            t = t + textbook_expert(orc, inp.sh13, inp.sh2, sh.I_sh, a, limit,
                                    inp.sh_h_gscale if act == A4 else None)
        out, rb = textbook_norm(orc, t, inp.gamma, sh.eps)
        assert np.array_equal(res["resid_out"][r], rb)
        assert np.allclose(res["out64"][r], out, rtol=1e-11, atol=1e-13)


def test_clamped_swiglu_closed_forms(orc):
    """Values the algebra fixes: e^-ln3 = 1/3, so silu(ln 3) = (3/4) ln 3; the
    clamp leaves values inside the limit alone, does not raise a low gate,
    makes the output constant in a gate above the limit and odd in up."""
    L = np.log(3.0)
    assert orc.swiglu(5.0, 7.0, L) == pytest.approx(0.75 * L * L, rel=1e-15)
    assert orc.swiglu(0.0, 0.9, L) == 0.0
    for g, u in [(0.3, -0.7), (-10.0, 1.0), (-4.0, -1.05), (L, L)]:
        assert orc.swiglu(g, u, L) == orc.swiglu(g, u, 0.0)
    for g in (L, 2.0, 50.0):
        assert orc.swiglu(g, 0.5, L) == orc.swiglu(L, 0.5, L)
    for u in (2.0, 9.0):
        assert orc.swiglu(0.4, u, L) == orc.swiglu(0.4, L, L)
        assert orc.swiglu(0.4, -u, L) == -orc.swiglu(0.4, u, L)
    # unclamped: no cap at all
    assert orc.swiglu(50.0, 9.0, 0.0) == pytest.approx(50.0 * 9.0, rel=1e-15)


def test_top_all_experts_is_dense_mixture(orc):
    sh = synth.custom_shape(M=2, H=64, E=4, k=4, I=32, routed_scale=1.0)
    inp, L = _layer(orc, sh, 8)
    res = L.rows(np.arange(2))
    for r in range(2):
        assert sorted(res["ids"][r]) == [0, 1, 2, 3]
        assert abs(res["w"][r].astype(np.float64).sum() - 1.0) < 1e-6
        a = _act(orc, inp, r)
        ys = [textbook_expert(orc, inp.w13.expert(e), inp.w2.expert(e), sh.I, a) for e in range(4)]
        for j in range(4):
            assert np.allclose(res["y"][r, j], ys[res["ids"][r, j]], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("wfmt", [synth.MXFP4, synth.NVFP4])
def test_w2_scale_doubling_doubles_y_exactly(orc, wfmt):
    sh = synth.custom_shape(M=3, H=128, E=4, k=2, I=64, wfmt=wfmt)
    inp = synth.make_inputs(sh, seed=10, pool_rows=512)
    base = orc.Layer(inp).rows(np.arange(3))
    if wfmt == synth.MXFP4:
        assert inp.w2.pool_scales.max() < 254
        inp.w2.pool_scales = inp.w2.pool_scales + 1
    else:
        inp.w2.gscale = inp.w2.gscale * np.float32(2)
    dbl = orc.Layer(inp).rows(np.arange(3))
    assert np.array_equal(dbl["y"], 2 * base["y"])


def test_gate_up_rows_are_gate_then_up(orc):
    """Swapping the gate and up halves of W13 changes h (silu is not
    symmetric), so the [gate; up] reading is observable."""
    sh = synth.custom_shape(M=1, H=64, E=1, k=1, I=32)
    inp = synth.make_inputs(sh, seed=3, pool_rows=512)
    m = inp.w13.expert(0)
    a = _act(orc, inp, 0)
    h = orc.gate_up(orc.Mat(m.fmt, m.packed, m.scales), sh.H, sh.I, a)
    W = dense(m)
    g, u = W[:32] @ a, W[32:] @ a
    assert np.allclose(h, g / (1 + np.exp(-g)) * u, rtol=1e-13, atol=1e-16)
    assert not np.allclose(h, u / (1 + np.exp(-u)) * g, rtol=1e-3)


def test_finalize_zero_experts_is_textbook_rmsnorm(orc):
    rng = np.random.default_rng(20)
    H, k = 256, 3
    res = synth._bf16_trunc(rng.standard_normal(H).astype(np.float32) * 3)
    gamma = synth._bf16_trunc(1 + 0.1 * rng.standard_normal(H).astype(np.float32))
    y = rng.standard_normal((k, H))
    out64, ob, ro = orc.finalize_row(y, np.zeros(k, np.float32), None, res, gamma, 1e-6)
    xv = bf16v(res)
    ref = xv / np.sqrt(np.mean(xv ** 2) + 1e-6) * bf16v(gamma)
    assert np.array_equal(ro, res)
    assert np.allclose(out64, ref, rtol=1e-13)


def test_finalize_constant_row_is_sign_times_gamma(orc):
    H = 128
    gamma = synth._bf16_trunc(np.linspace(0.5, 1.5, H).astype(np.float32))
    for v in (-3.0, 0.25, 7.0):
        res = synth._bf16_trunc(np.full(H, v, np.float32))
        out64, _, _ = orc.finalize_row(np.zeros((1, H)), np.zeros(1, np.float32), None, res, gamma, 1e-6)
        expect = np.sign(v) * bf16v(gamma) / np.sqrt(1 + 1e-6 / v ** 2)
        assert np.allclose(out64, expect, rtol=1e-13)


def test_finalize_weights_and_shared_add(orc):
    rng = np.random.default_rng(21)
    H, k = 64, 4
    res = synth._bf16_trunc(rng.standard_normal(H).astype(np.float32))
    gamma = synth._bf16_trunc(np.ones(H, np.float32))
    y = rng.standard_normal((k, H))
    ysh = rng.standard_normal(H)
    w = rng.random(k).astype(np.float32)
    out64, ob, ro = orc.finalize_row(y, w, ysh, res, gamma, 1e-6)
    t = bf16v(res) + ysh + w.astype(np.float64) @ y
    ref, rb = textbook_norm(orc, t, gamma, 1e-6)
    assert np.array_equal(ro, rb)
    assert np.allclose(out64, ref, rtol=1e-13)
    assert np.array_equal(ob, orc.bf16_rne_n(out64))


def test_rows_subset_and_own_logits(orc):
    sh = synth.custom_shape(M=6, H=128, E=8, k=2, I=32, bias="normal:0.01")
    inp = synth.make_inputs(sh, seed=12, pool_rows=1024)
    L = orc.Layer(inp)
    full = L.rows(np.arange(6))
    sub = L.rows(np.array([4, 1]))
    assert np.array_equal(sub["out64"], full["out64"][[4, 1]])
    lg = orc.router_logits(inp.x, inp.Wr).astype(np.float32)
    given = L.rows(np.arange(6), logits=lg)
    assert np.array_equal(given["out64"], full["out64"])
    assert np.array_equal(given["ids"], full["ids"])


def test_nan_scale_propagates(orc):
    sh = synth.custom_shape(M=1, H=64, E=1, k=1, I=32)
    inp = synth.make_inputs(sh, seed=2, pool_rows=256)
    inp.w2.pool_scales = inp.w2.pool_scales.copy()
    inp.w2.pool_scales[:, 0] = 0xFF  # E8M0 NaN in every W2 row
    res = orc.Layer(inp).rows(np.array([0]))
    assert np.isnan(res["y"]).all() and np.isnan(res["out64"]).all()
