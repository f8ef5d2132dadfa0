"""Pins of the oracle's static-FP8 shared expert (README Qwen3.5 slot table,
row "route_shared": the shared gate/up on static FP8; sgl-nvidia-mega PR #33,
appended table, row "shared act quant": SiLU-and-mul fused with the static FP8
quant of the down input).  Each check reaches the expected value by another
route than the oracle's: torch's float8_e4m3fn cast after numpy's fp32
division, exact dyadic matrix products in numpy, torch's bf16 rounding and
silu, and invariances the arithmetic fixes (a power-of-two change of a static
input scale leaves every product unchanged; a doubled weight scale doubles the
output exactly)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_scaled_fp4_sigmoid_amd import synth


def bf16v(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3v(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3(q32: np.ndarray) -> np.ndarray:
    """E4M3 codes of fp32 values by torch's cast (round to nearest even; it
    does not saturate, so only values up to 448 in magnitude are passed)."""
    return torch.from_numpy(np.ascontiguousarray(q32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def quant_all(orc, v, s):
    return np.array([orc.fp8s_quant(float(x), s) for x in np.asarray(v, np.float32)], np.uint8)


@pytest.mark.parametrize("s", [2.0 ** -4, 1.0, 8.0, 0.0123, 3.7])
def test_quant_is_e4m3_of_the_fp32_quotient(orc, s):
    """Every finite bf16 value whose quotient is in range: the code is torch's
    E4M3 of numpy's fp32 quotient; beyond 448 it saturates with the sign."""
    rng = np.random.default_rng(int(s * 1000))
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]            # finite bf16 only
    bits = rng.choice(bits, 6000, replace=False).astype(np.uint16)
    v = bf16v(bits).astype(np.float32)
    with np.errstate(over="ignore"):
        q32 = v / np.float32(s)                           # numpy: IEEE fp32 division
    got = quant_all(orc, v, s)
    inr = np.abs(q32) <= 448
    assert np.array_equal(got[inr], torch_e4m3(q32[inr]))
    sat = ~inr
    assert np.array_equal(got[sat], np.where(np.signbit(q32[sat]), 0xFE, 0x7E).astype(np.uint8))
    assert inr.sum() > 1000


def test_quant_takes_the_fp32_quotient_not_the_exact_one(orc):
    """Values whose exact quotient lies just above an E4M3 midpoint while its
    fp32 rounding lands on the midpoint itself: the fp32 quotient ties to the
    even code, the exact one would round up.  Found by a search over bf16
    values and fp32 scales with exact rational arithmetic."""
    found = 0
    for mant in range(128):
        v = np.float32(1.0 + mant / 128.0)                # a bf16 value in [1, 2)
        for m in (1.0625, 1.1875, 1.3125, 1.4375):        # midpoints between E4M3 values in [1, 2)
            ulp = Fraction(1, 1 << 23)
            target = Fraction(m) + ulp / 4                # inside (m, m + ulp / 2)
            s = np.float32(float(Fraction(float(v)) / target))
            for cand in (s, np.nextafter(s, np.float32(0)), np.nextafter(s, np.float32(9))):
                exact = Fraction(float(v)) / Fraction(float(cand))
                if not (Fraction(m) < exact < Fraction(m) + ulp / 2):
                    continue
                assert np.float32(v) / cand == np.float32(m)  # numpy's fp32 quotient is the midpoint
                lo = int(torch_e4m3(np.array([m - 0.0625], np.float32))[0])
                hi = int(torch_e4m3(np.array([m + 0.0625], np.float32))[0])
                even = lo if lo % 2 == 0 else hi
                assert orc.fp8s_quant(float(v), float(cand)) == even
                found += 1
    assert found >= 10


def test_quant_specials_and_round_trip(orc):
    s = 0.25
    assert orc.fp8s_quant(float("nan"), s) in (0x7F, 0xFF)
    assert orc.fp8s_quant(float("inf"), s) == 0x7E
    assert orc.fp8s_quant(float("-inf"), s) == 0xFE
    assert orc.fp8s_quant(0.0, s) == 0x00
    assert orc.fp8s_quant(-0.0, s) == 0x80
    assert orc.fp8s_quant(1e30, s) == 0x7E
    assert orc.fp8s_quant(455 * s, s) == 0x7E          # between 448 and 464: rounds down to 448
    # every finite code survives value * s -> quant for power-of-two s
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for sp in (2.0 ** -3, 1.0, 4.0):
        vals = e4m3v(codes) * sp
        assert np.array_equal(quant_all(orc, vals, sp), codes)


def _fp8s_mat(orc, rng, N, K, s_w, small=True):
    """A static-FP8 matrix whose codes have small dyadic values (products and
    sums then stay exact in fp64)."""
    pool = np.array([0x30, 0x38, 0x3C, 0x40, 0x44, 0xB0, 0xB8, 0xBC, 0xC0, 0x00], np.uint8)  # 0.5..3, signs, 0
    codes = rng.choice(pool, size=(N, K)).astype(np.uint8)
    return codes, orc.Mat(orc.ORC_FP8S, codes, None, s_w)


def test_gate_up_textbook_on_exact_values(orc):
    """Inputs that are E4M3 values times a power-of-two scale (so the input
    quant is exact) and dyadic weights: g, u are the exact products, rounded
    to bf16 by torch; h is torch's silu(g) * u in fp64, rounded to bf16."""
    rng = np.random.default_rng(1)
    H, I, s_in, s_w = 64, 16, 0.5, 2.0 ** -5
    codes, m = _fp8s_mat(orc, rng, 2 * I, H, s_w)
    xc = rng.choice(np.array([0x38, 0x30, 0x40, 0xB8, 0x44, 0x2C], np.uint8), H)
    x = torch_bf16_bits(e4m3v(xc) * s_in)
    h, gu = orc.gate_up_fp8s(m, H, I, x, s_in)
    W = e4m3v(codes) * s_w
    G = s_in * (W @ e4m3v(xc))                             # exact: dyadic values, short sums
    assert np.array_equal(gu, torch_bf16_bits(G))
    g, u = bf16v(gu[:I]), bf16v(gu[I:])
    hh = torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)
    assert np.array_equal(h, torch_bf16_bits(hh.numpy()))


def test_gate_up_scale_invariances(orc):
    """A power-of-two change of the static input scale shifts every code's
    exponent and is undone by the output scale: g, u, h unchanged.  A doubled
    weight scale doubles g and u exactly."""
    rng = np.random.default_rng(2)
    H, I = 256, 32
    sh = synth.custom_shape(M=1, H=H, E=1, k=1, I=64, sfmt=synth.FP8S, I_sh=I)
    inp = synth.make_inputs(sh, seed=4, pool_rows=256)
    xf = rng.standard_normal(H).astype(np.float32)
    xf = np.where(np.abs(xf) < 0.05, np.float32(0.05) * np.sign(xf + 1e-9), xf).astype(np.float32)
    x = synth._bf16_trunc(xf)
    s_in = float(np.float32(np.abs(bf16v(x)).max()) / np.float32(448))
    m = orc.Mat.from_synth(inp.sh13)
    h0, gu0 = orc.gate_up_fp8s(m, H, I, x, s_in)
    for f in (2.0, 4.0, 16.0):
        h1, gu1 = orc.gate_up_fp8s(m, H, I, x, s_in * f)
        assert np.array_equal(gu1, gu0) and np.array_equal(h1, h0)
    m2 = orc.Mat(orc.ORC_FP8S, inp.sh13.packed, None, 2 * inp.sh13.gscale)
    _, gu2 = orc.gate_up_fp8s(m2, H, I, x, s_in)
    assert np.array_equal(bf16v(gu2), 2 * bf16v(gu0))


def test_down_textbook_and_invariances(orc):
    rng = np.random.default_rng(3)
    H, I, s_in, s_w = 48, 64, 0.25, 2.0 ** -4
    codes, m = _fp8s_mat(orc, rng, H, I, s_w)
    hc = rng.choice(np.array([0x38, 0x30, 0x40, 0xB8, 0x44, 0x00, 0x2C], np.uint8), I)
    h = torch_bf16_bits(e4m3v(hc) * s_in)
    y, hq = orc.down_fp8s(m, H, I, h, s_in)
    assert np.array_equal(hq, hc)
    assert np.array_equal(y, s_in * ((e4m3v(codes) * s_w) @ e4m3v(hc)))
    # h of general values: the codes are the static quant of each value
    hr = synth._bf16_trunc(rng.standard_normal(I).astype(np.float32))
    y1, hq1 = orc.down_fp8s(m, H, I, hr, 0.01)
    assert np.array_equal(hq1, quant_all(orc, bf16v(hr), 0.01))
    hr = np.where(np.abs(bf16v(hr)) < 0.05, synth._bf16_trunc(np.array([0.05], np.float32))[0], hr).astype(np.uint16)
    y1, _ = orc.down_fp8s(m, H, I, hr, 0.01)
    y2, _ = orc.down_fp8s(m, H, I, hr, 0.02)           # codes one binade down, output scale up
    assert np.array_equal(y1, y2)
    m2 = orc.Mat(orc.ORC_FP8S, codes, None, 2 * s_w)
    y3, _ = orc.down_fp8s(m2, H, I, hr, 0.01)
    assert np.array_equal(y3, 2 * y1)


@pytest.mark.parametrize("wfmt,act,limit", [(synth.MXFP4, synth.ACT_MXFP8, 0.0), (synth.NVFP4, synth.ACT_NVFP4, 0.0),
                                            (synth.NVFP4, synth.ACT_MXFP8, 0.4)])
def test_layer_shared_output_is_the_standalone_fp8s_expert(orc, wfmt, act, limit):
    """The layer's shared-expert output is the static-FP8 expert applied to
    the bf16 layer input with its gate/up scale and h with its down scale (the
    two static scales are not interchangeable), clamped with the layer's
    limit; the finalize adds it."""
    sh = synth.custom_shape(M=3, H=256, E=4, k=2, I=128, wfmt=wfmt, sfmt=synth.FP8S, I_sh=64, act_fmt=act,
                            swiglu_limit=limit)
    inp = synth.make_inputs(sh, seed=12, pool_rows=512)
    assert inp.sh_in13 > 0 and inp.sh_in2 > 0 and inp.sh_in13 != inp.sh_in2
    res = orc.Layer(inp).rows(np.arange(sh.M))
    m13, m2 = orc.Mat.from_synth(inp.sh13), orc.Mat.from_synth(inp.sh2)
    for r in range(sh.M):
        h, _ = orc.gate_up_fp8s(m13, sh.H, sh.I_sh, inp.x[r], inp.sh_in13, limit)
        y, _ = orc.down_fp8s(m2, sh.H, sh.I_sh, h, inp.sh_in2)
        assert np.array_equal(res["y_sh"][r], y)
        ref = orc.finalize_row(res["y"][r], res["w"][r], y, inp.x[r], inp.gamma, sh.eps)
        assert np.array_equal(res["resid_out"][r], ref[2])
    if limit > 0:  # the clamp reaches the shared expert: unclamped differs
        h_c, _ = orc.gate_up_fp8s(m13, sh.H, sh.I_sh, inp.x[0], inp.sh_in13, limit)
        h_u, _ = orc.gate_up_fp8s(m13, sh.H, sh.I_sh, inp.x[0], inp.sh_in13, 0.0)
        assert not np.array_equal(h_c, h_u)


def test_layer_rejects_missing_static_scales(orc):
    sh = synth.custom_shape(M=2, H=128, E=2, k=1, I=64, sfmt=synth.FP8S, I_sh=64)
    inp = synth.make_inputs(sh, seed=13, pool_rows=256)
    inp.sh_in2 = 0.0
    with pytest.raises(ValueError):
        orc.Layer(inp).rows(np.arange(2))
