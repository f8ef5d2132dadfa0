"""Pins of the oracle's number formats and encoders against things other than
itself: the OCP MX v1.0 value tables (tests/golden), torch's CPU float8
dtypes, exhaustive nearest-value searches and closed-form invariants."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch


def _golden(golden_dir):
    rows = {}
    with open(os.path.join(golden_dir, "ocp_mx_format_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, code, val = line.split()
            rows.setdefault(fmt, []).append((int(code, 16), val))
    return rows


def _same(a: float, b: str) -> bool:
    if b == "nan":
        return math.isnan(a)
    bv = float(b)
    return a == bv and math.copysign(1, a) == math.copysign(1, bv)


def test_tables_match_ocp_golden(orc, golden_dir):
    g = _golden(golden_dir)
    tabs = {"e2m1": orc.e2m1_table(), "e4m3": orc.e4m3_table(), "e8m0": orc.e8m0_table()}
    assert len(g["e2m1"]) == 16
    for fmt, rows in g.items():
        for code, val in rows:
            assert _same(float(tabs[fmt][code]), val), (fmt, hex(code), tabs[fmt][code], val)


def test_e4m3_table_matches_torch_all_codes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = orc.e4m3_table()
    nan_ref, nan_mine = np.isnan(ref), np.isnan(mine)
    assert (nan_ref == nan_mine).all()
    assert set(np.nonzero(nan_mine)[0]) == {0x7F, 0xFF}
    assert (ref[~nan_ref] == mine[~nan_mine]).all()
    assert (np.signbit(ref[~nan_ref]) == np.signbit(mine[~nan_mine])).all()


def test_e8m0_table_matches_torch_all_codes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = orc.e8m0_table()
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert (ref[:255] == mine[:255]).all()
    # every code is an exact power of two
    for c in range(255):
        m, e = math.frexp(mine[c])
        assert m == 0.5 and e - 1 == c - 127


def test_e2m1_table_closed_form(orc):
    # the 8 magnitudes are exactly the values 2^(e-1) * (1 + m/2) (e>0) and m/2 (e=0)
    t = orc.e2m1_table()
    assert sorted(set(np.abs(t))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert all(t[c] == -t[c ^ 8] for c in range(16))
    assert np.signbit(t[8]) and not np.signbit(t[0])


def _finite_e4m3(orc):
    t = orc.e4m3_table()
    codes = np.array([c for c in range(128) if not math.isnan(t[c])])
    return codes, t[codes]


def _e4m3_bruteforce(v: np.ndarray, codes, vals) -> np.ndarray:
    """Nearest finite E4M3 magnitude (codes 0..0x7E), ties to the even code,
    sign copied; equivalent to RNE with saturation at 448."""
    out = np.empty(v.shape[0], np.uint8)
    a = np.abs(v)
    for s in range(0, v.shape[0], 8192):
        aa = a[s:s + 8192, None]
        d = np.abs(aa - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among tied candidates prefer the even code
        even = (codes[None, :] & 1) == 0
        pick_even = (cand & even).any(axis=1)
        choose = np.where(pick_even[:, None], cand & even, cand)
        idx = choose.argmax(axis=1)
        out[s:s + 8192] = codes[idx]
    return out | (np.signbit(v).astype(np.uint8) << 7)


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def test_e4m3_encoder_bruteforce_all_bf16_times_scales(orc):
    """Every finite bf16 value times every power of two that lands it in or
    near the E4M3 range, against an exhaustive nearest-of-codes search."""
    codes, vals = _finite_e4m3(orc)
    base = _all_finite_bf16()
    rng = np.random.default_rng(0)
    for t in range(-140, 141, 7):
        v = np.ldexp(base, t)
        v = v[np.isfinite(v) & (np.abs(v) < 2.0 ** 12)]
        if v.size > 20000:
            v = rng.choice(v, 20000, replace=False)
        got = orc.e4m3_rne_sat_n(v)
        ref = _e4m3_bruteforce(v, codes, vals)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (t, v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_encoder_ties_and_saturation(orc):
    # exact midpoints round to the even code
    assert orc.e4m3_rne_sat(1.0625) == 0x38   # between 1 (0x38) and 1.125 (0x39)
    assert orc.e4m3_rne_sat(1.1875) == 0x3A   # between 1.125 and 1.25 -> 1.25 (even)
    assert orc.e4m3_rne_sat(464.0) == 0x7E    # between 448 and (absent) 480
    assert orc.e4m3_rne_sat(1e30) == 0x7E     # saturates
    assert orc.e4m3_rne_sat(-1e30) == 0xFE
    assert orc.e4m3_rne_sat(2.0 ** -10) == 0x00   # half of the smallest subnormal: tie to 0
    assert orc.e4m3_rne_sat(3 * 2.0 ** -10) == 0x02  # 1.5 quanta -> 2 (even)
    assert orc.e4m3_rne_sat(-0.0) == 0x80
    assert orc.e4m3_rne_sat(float("nan")) == 0x7F


def test_e4m3_encoder_matches_torch_in_range(orc):
    """torch's float8_e4m3fn cast is RNE; it does not saturate, so compare
    only values whose magnitude stays below 464."""
    base = _all_finite_bf16()
    for t in (-12, -6, -3, 0, 3):
        v = np.ldexp(base, t)
        v = v[np.isfinite(v) & (np.abs(v) < 464.0)]
        ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(orc.e4m3_rne_sat_n(v), ref), t


def _bf16_bruteforce(v: float) -> int:
    """Nearest bf16 by exact rational comparison, ties to even mantissa."""
    f32 = np.array([abs(v)], np.float32).view(np.uint32)[0]
    base = int(f32 >> 16)
    best = None
    for b in range(max(base - 2, 0), min(base + 3, 0x7F80) + 1):
        val = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        d = abs(Fraction(abs(v)) - Fraction(val))
        key = (d, b & 1)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1] | (0x8000 if math.copysign(1, v) < 0 else 0)


def test_bf16_rne_bruteforce(orc):
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-100, 100, 3000)))
    # exact ties: midpoints between consecutive bf16 values
    for b in rng.integers(0x0080, 0x7F00, 500):
        lo = float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(int(b) + 1) << 16], np.uint32).view(np.float32)[0])
        vals.append((lo + hi) / 2)
        vals.append(-(lo + hi) / 2)
    got = orc.bf16_rne_n(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == _bf16_bruteforce(v), (v, hex(int(g)))


def test_bf16_rne_specials(orc):
    assert orc.bf16_rne(float("inf")) == 0x7F80
    assert orc.bf16_rne(-float("inf")) == 0xFF80
    assert orc.bf16_rne(2.0 ** 200) == 0x7F80
    assert orc.bf16_rne(-0.0) == 0x8000
    assert orc.bf16_rne(2.0 ** -133) == 0x0001   # smallest subnormal
    assert orc.bf16_rne(2.0 ** -134) == 0x0000   # tie to even (0)
    assert orc.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80  # tie -> even
    assert orc.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert math.isnan(orc.bf16_value(orc.bf16_rne(float("nan"))))


def _bf16_from_f32(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_mxfp8_scale_rule_invariants(orc):
    """OCP MX rule: after scaling, the block's largest |q| lies in [256, 448]
    (E4M3 max exponent 8); scaling the input by 2^t moves only the scale code."""
    rng = np.random.default_rng(2)
    x = _bf16_from_f32(rng.standard_normal((64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1))))
    q, s = orc.mxfp8_quant_bf16(x)
    e4 = orc.e4m3_table()
    qv = np.abs(e4[q]).reshape(64, 16, 32)
    mx = qv.max(axis=2)
    assert ((mx >= 256) & (mx <= 448)).all()
    # scale code = floor(log2 amax) - 8 + 127, from the bf16 exponent field
    xb = x.reshape(64, 16, 32)
    amax_bits = (xb & 0x7FFF).max(axis=2).astype(np.int64)
    assert (s.astype(np.int64) == (amax_bits >> 7) - 127 - 8 + 127).all()
    # power-of-two scaling shifts only the scale
    x2 = _bf16_from_f32(((x.astype(np.uint32) << 16).view(np.float32)) * np.float32(2.0 ** 5))
    q2, s2 = orc.mxfp8_quant_bf16(x2)
    assert np.array_equal(q2, q) and np.array_equal(s2.astype(int), s.astype(int) + 5)


def test_mxfp8_elements_are_nearest(orc):
    """Every element code is the RNE-saturated E4M3 of x / 2^(scale-127)."""
    codes, vals = _finite_e4m3(orc)
    rng = np.random.default_rng(3)
    x = _bf16_from_f32(rng.standard_normal((16, 256)) * 3)
    q, s = orc.mxfp8_quant_bf16(x)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sc = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    ref = _e4m3_bruteforce(np.ldexp(xv, -sc).ravel(), codes, vals).reshape(q.shape)
    assert np.array_equal(q, ref)


def test_mxfp8_roundtrip_on_representable(orc):
    """quantize -> dequantize is the identity on blocks that are already
    E4M3 values times 2^t with a block max in [256, 448]."""
    rng = np.random.default_rng(4)
    codes, vals = _finite_e4m3(orc)
    for _ in range(200):
        t = int(rng.integers(-100, 100))
        c = rng.choice(codes, 32)
        c[rng.integers(32)] = rng.choice([0x70, 0x74, 0x78, 0x7A, 0x7E])  # max in [256, 448]... or 128-240
        v = orc.e4m3_table()[c] * (1 - 2 * rng.integers(0, 2, 32))
        if np.abs(v).max() < 256:
            v[np.argmax(np.abs(v))] = 256.0
        v = np.ldexp(v, t)
        q, s = orc.mxfp8_quant_f64(v[None, :])
        back = orc.mxfp8_dequant(q, s)[0]
        assert np.array_equal(back, v), t


def test_mxfp8_zero_and_special_blocks(orc):
    z = np.zeros((1, 32))
    z[0, 3] = -0.0
    q, s = orc.mxfp8_quant_f64(z)
    assert s[0, 0] == 0 and set(q[0]) <= {0x00, 0x80} and q[0, 3] == 0x80
    v = np.ones((1, 32))
    v[0, 5] = np.nan
    q, s = orc.mxfp8_quant_f64(v)
    assert s[0, 0] == 0xFF and (q[0] & 0x7F == 0x7F).all()
    v = np.ones((1, 32))
    v[0, 7] = -np.inf
    q, s = orc.mxfp8_quant_f64(v)
    assert s[0, 0] == 0xFF and q[0, 7] == 0xFF
    # bf16 subnormal block: shared exponent clamps at -127
    x = np.full((1, 32), 0x0001, np.uint16)  # 2^-133
    q, s = orc.mxfp8_quant_bf16(x)
    assert s[0, 0] == 0 and orc.e4m3_table()[q[0, 0]] == 2.0 ** -6


# ---- NVFP4 activations --------------------------------------------------------

def _e2m1_by_quantum(a: np.ndarray) -> np.ndarray:
    """E2M1 magnitude of |a| as ordinary rounding to the format's spacing:
    0.5 below 2, 1 below 4, 2 above; numpy's rint rounds halves to even
    multiples, which are the even codes; saturating at 6."""
    a = np.abs(a.astype(np.float64))
    q = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    return np.minimum(np.rint(a / q) * q, 6.0)


E2M1_MAG = [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_encoder_matches_quantum_rounding(orc):
    # every multiple of 1/64 in [0, 8], the midpoints included, and random values
    rng = np.random.default_rng(7)
    vals = np.concatenate([np.arange(0, 8.0001, 1 / 64), rng.random(4000) * 9]).astype(np.float32)
    for v in vals:
        for sgn in (1.0, -1.0):
            c = orc.e2m1_rne_sat(sgn * float(v))
            assert (c >> 3) == (1 if sgn < 0 else 0)
            assert E2M1_MAG[c & 7] == _e2m1_by_quantum(np.array([v]))[0], (v, c)
    assert orc.e2m1_rne_sat(-0.0) == 8 and orc.e2m1_rne_sat(1e30) == 7


def _nvfp4_block_independent(v: np.ndarray, g: float):
    """The stated rule re-derived with numpy fp32 arithmetic and torch's E4M3."""
    v = v.astype(np.float32)
    g = np.float32(g)
    if not np.all(np.isfinite(v)):
        return np.zeros(8, np.uint8), 0x7F
    amax = np.max(np.abs(v))
    s = np.float32(amax) / np.float32(np.float32(6.0) * g)
    s = min(float(s), 448.0)
    sc = int(torch.tensor([s], dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    sd = np.float32(torch.tensor([sc], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)[0])
    if sd == 0:
        return np.zeros(8, np.uint8), sc
    d = np.float32(sd * g)
    qv = (v / d).astype(np.float32)
    mag = _e2m1_by_quantum(qv)
    codes = np.array([E2M1_MAG.index(m) for m in mag]) | (np.signbit(qv).astype(int) << 3)
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), sc


def test_nvfp4_block_rule_independent(orc):
    rng = np.random.default_rng(8)
    for t in range(3000):
        g = float(np.float32(np.exp2(rng.uniform(-12, 2))))
        v = (rng.standard_normal(16) * np.exp2(rng.uniform(-8, 8))).astype(np.float32)
        if t % 7 == 0:
            v[rng.integers(16)] = 0.0
        if t % 11 == 0:
            v = v * np.float32(1e4)          # scales saturate at 448
        q, s = orc.nvfp4_quant_f32(v[None, :], g)
        rq, rs = _nvfp4_block_independent(v, g)
        assert s[0, 0] == rs and np.array_equal(q[0], rq), (t, v, g)


def test_nvfp4_roundtrip_on_representable(orc):
    """Values e2m1 * E4M3 * g whose block holds a +-6 element decode exactly
    (g a power of two keeps every fp32 step exact)."""
    rng = np.random.default_rng(9)
    e4 = torch.arange(1, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for _ in range(500):
        g = float(np.exp2(rng.integers(-10, 3)))
        sd = float(e4[rng.integers(len(e4))])
        mags = np.array(E2M1_MAG)[rng.integers(0, 8, 16)]
        mags[rng.integers(16)] = 6.0
        v = (mags * np.where(rng.random(16) < 0.5, -1, 1) * sd * g).astype(np.float32)
        q, s = orc.nvfp4_quant_f32(v[None, :], g)
        back = orc.nvfp4_dequant(q, s, g)[0]
        assert np.array_equal(back, v.astype(np.float64)), (v, back)


def test_nvfp4_zero_special_and_saturated_blocks(orc):
    z = np.zeros((1, 16), np.float32)
    q, s = orc.nvfp4_quant_f32(z, 0.25)
    assert s[0, 0] == 0 and not q.any()
    for bad in (np.nan, np.inf, -np.inf):
        v = np.ones((1, 32), np.float32)
        v[0, 3] = bad
        q, s = orc.nvfp4_quant_f32(v, 1.0)
        assert s[0, 0] == 0x7F and not q[0, :8].any()       # the block holding it
        # the other block: amax 1, s = 1/6 = 2^-3 * 1.33.., nearest E4M3 2^-3 * 1.375 = code 0x23
        assert s[0, 1] == 0x23
        assert np.isnan(orc.nvfp4_dequant(q, s, 1.0)[0, :16]).all()
    # amax far above 6 * 448 * g: scale 448, elements clip at 6
    v = np.full((1, 16), 1e6, np.float32)
    q, s = orc.nvfp4_quant_f32(v, 1.0)
    assert s[0, 0] == 0x7E and np.all(q == 0x77)
    # a block whose scale underflows E4M3 (below half of 2^-9) encodes zeros
    v = np.full((1, 16), 1e-6, np.float32)
    q, s = orc.nvfp4_quant_f32(v, 1.0)
    assert s[0, 0] == 0 and not q.any()


def test_nvfp4_bf16_rows_equal_f32_rows(orc):
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((5, 256)).astype(np.float32))
    xb = ((x.view(np.uint32) >> 16).astype(np.uint16))
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    a = orc.nvfp4_quant_bf16(xb, 0.003)
    b = orc.nvfp4_quant_f32(xf, 0.003)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
