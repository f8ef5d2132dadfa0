"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake (a dropped term, a wrong sign, a swapped index, a wrong block size,
...) into a private copy of the oracle source, builds it on the CPU, and runs
the oracle pin suite against it in a subprocess; the suite has to fail."""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_route.py", "tests/test_oracle_layer.py",
        "tests/test_oracle_fp8s.py"]

MUTANTS = {
    "up rows read from the gate half": ("orc_mat_row(w13, H, I + n, wrow);", "orc_mat_row(w13, H, n, wrow);"),
    "silu dropped": ("return (g / (1.0 + exp(-g))) * u;", "return g * u;"),
    "clamped gate capped from below too": ("        if (g > limit)\n            g = limit;\n",
                                           "        if (g > limit)\n            g = limit;\n        if (g < -limit)\n            g = -limit;\n"),
    "clamped up one-sided": ("        if (u < -limit)\n            u = -limit;\n", ""),
    "clamped gate not capped": ("        if (g > limit)\n            g = limit;\n", ""),
    "clamp left out of the routed experts": ("expert_fp4(&L->w13[e], &L->w2[e], H, I, a, L->swiglu_limit,",
                                             "expert_fp4(&L->w13[e], &L->w2[e], H, I, a, 0.0,"),
    "clamp left out of the shared expert": ("expert_fp4(&L->sh13, &L->sh2, H, L->I_sh, a, L->swiglu_limit,",
                                            "expert_fp4(&L->sh13, &L->sh2, H, L->I_sh, a, 0.0,"),
    "clamp left out of the bf16 shared expert": ("L->x + (size_t)r * H, L->swiglu_limit, h);",
                                                 "L->x + (size_t)r * H, 0.0, h);"),
    "sigmoid sign flipped": ("s[e] = 1.0 / (1.0 + exp(-(double)logits_row[e]));",
                             "s[e] = 1.0 / (1.0 + exp((double)logits_row[e]));"),
    "bias leaks into weights": ("w[j] = (float)((scale * s[ids[j]]) / sum);",
                                "w[j] = (float)((scale * key[ids[j]]) / sum);"),
    "ties to the higher id": ("if (best < 0 || key[e] > key[best])", "if (best < 0 || key[e] >= key[best])"),
    "routed scale dropped": ("w[j] = (float)((scale * s[ids[j]]) / sum);", "w[j] = (float)((s[ids[j]]) / sum);"),
    "MX shared exponent off by one": ("shared = (e - 1) - 8;", "shared = (e - 1) - 7;"),
    "nibble order swapped": ("int code = (k & 1) ? (byte >> 4) : (byte & 15);",
                             "int code = (k & 1) ? (byte & 15) : (byte >> 4);"),
    "NVFP4 block of 32": ("scale = T_E4M3[m->scales[(size_t)n * (K / 16) + k / 16]] * (double)m->gscale;",
                          "scale = T_E4M3[m->scales[(size_t)n * (K / 16) + k / 32]] * (double)m->gscale;"),
    "NVFP4 global dropped": ("scale = T_E4M3[m->scales[(size_t)n * (K / 16) + k / 16]] * (double)m->gscale;",
                             "scale = T_E4M3[m->scales[(size_t)n * (K / 16) + k / 16]];"),
    "E2M1 subnormal wrong": ("double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m * 0.5, e - 1);",
                             "double mag = (e == 0) ? m * 1.0 : ldexp(1.0 + m * 0.5, e - 1);"),
    "E4M3 bias 8": ("mag = ldexp(1.0 + m / 8.0, e - 7);", "mag = ldexp(1.0 + m / 8.0, e - 8);"),
    "round toward zero": ("return rint(a / quantum) * quantum;", "return floor(a / quantum) * quantum;"),
    "requant skipped before down": ("orc_down(w2, H, I, hd, y);", "orc_down(w2, H, I, h, y);"),
    "bf16 shared intermediate not rounded": ("h[n] = orc_bf16_value(orc_bf16_rne(h[n]));", "h[n] = h[n];"),
    "residual dropped": ("double t = orc_bf16_value(residual[c]) + (y_sh ? y_sh[c] : 0.0);",
                         "double t = (y_sh ? y_sh[c] : 0.0);"),
    "shared expert dropped": ("double t = orc_bf16_value(residual[c]) + (y_sh ? y_sh[c] : 0.0);",
                              "double t = orc_bf16_value(residual[c]);"),
    "RMS without the mean": ("double inv = 1.0 / sqrt(ss / H + eps);", "double inv = 1.0 / sqrt(ss + eps);"),
    "norm on the unrounded sum": ("rr[c] = orc_bf16_value(rb);", "rr[c] = t;"),
    "tiles of 7": ("tile_rows[t] = (n - 8 * i < 8) ? (n - 8 * i) : 8;", "tile_rows[t] = (n - 8 * i < 8) ? (n - 8 * i) : 7;"),
    "bucket rows descending": ("        for (int r = 0; r < M; ++r)\n            for (int j = 0; j < k; ++j)\n                if (ids[(size_t)r * k + j] == e)",
                               "        for (int r = M - 1; r >= 0; --r)\n            for (int j = 0; j < k; ++j)\n                if (ids[(size_t)r * k + j] == e)"),
    "E2M1 ties to the larger code": ("if (dc < db || (dc == db && (c & 1) == 0))", "if (dc < db || dc == db)"),
    "NVFP4 scale without the 6": ("const float t = 6.0f * g;", "const float t = g;"),
    "NVFP4 codes ignore the global": ("const float d = sd * g;", "const float d = sd;"),
    "NVFP4 nibbles swapped in the encoder": ("q8[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));",
                                            "q8[i] = (uint8_t)(codes[2 * i + 1] | (codes[2 * i] << 4));"),
    "NVFP4 nibbles swapped in the decoder": ("const int code = (i & 1) ? (q[i / 2] >> 4) : (q[i / 2] & 15);",
                                            "const int code = (i & 1) ? (q[i / 2] & 15) : (q[i / 2] >> 4);"),
    "NVFP4 non-finite block kept": ("        if (!isfinite(v[i]))\n            finite = 0;\n        else if",
                                    "        if (0)\n            finite = 0;\n        else if"),
    "W4A4 input quantized as MXFP8": ("    if (L->act_fmt == ORC_ACT_NVFP4) {\n        orc_nvfp4_quant_bf16(",
                                      "    if (0) {\n        orc_nvfp4_quant_bf16("),
    "W4A4 h requant without its global": ("orc_nvfp4_quant_f32(hf, 1, I, h_g, q, s);",
                                          "orc_nvfp4_quant_f32(hf, 1, I, 1.0f, q, s);"),
    "W4A4 shared h with a routed global": ("L->act_fmt, L->sh_h_gscale, ysh,", "L->act_fmt, L->h_gscale[0], ysh,"),
    "E4M3 not saturating": ("    if (r > 448.0)\n        r = 448.0;\n", ""),
    "static FP8 multiplies by its scale": ("const float q = v / s_in;", "const float q = v * s_in;"),
    "static FP8 quotient in fp64": ("return orc_e4m3_rne_sat((double)q);",
                                    "(void)q;\n    return orc_e4m3_rne_sat((double)v / (double)s_in);"),
    "static FP8 gate/up without its input scale": ("const uint16_t gb = orc_bf16_rne(g * (double)s_in);",
                                                   "const uint16_t gb = orc_bf16_rne(g);"),
    "static FP8 gate/up outputs not rounded to bf16": (
        "h[n] = orc_bf16_rne(orc_swiglu(orc_bf16_value(gb), orc_bf16_value(ub), limit));",
        "h[n] = orc_bf16_rne(orc_swiglu(g * (double)s_in, u * (double)s_in, limit));"),
    "static FP8 down without its input scale": ("        y[c] *= (double)s_in;\n", ""),
    "static FP8 weight scale dropped": ("out[k] = T_E4M3[m->packed[(size_t)n * K + k]] * (double)m->gscale;",
                                        "out[k] = T_E4M3[m->packed[(size_t)n * K + k]];"),
    "static FP8 shared input scales swapped": ("L->x + (size_t)r * H, L->sh_in13, L->swiglu_limit, h, NULL);",
                                               "L->x + (size_t)r * H, L->sh_in2, L->swiglu_limit, h, NULL);"),
    "clamp left out of the static FP8 shared expert": ("L->x + (size_t)r * H, L->sh_in13, L->swiglu_limit, h, NULL);",
                                                       "L->x + (size_t)r * H, L->sh_in13, 0.0, h, NULL);"),
}


def _run(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name!r} not found"
    mutated = src.replace(old, new, 1)
    d = os.path.join(tmp, "m%d" % abs(hash(name)))
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, "moe_oracle.c")
    open(c, "w").write(mutated)
    for hdr in ("moe_oracle.h",):
        open(os.path.join(d, hdr), "w").write(open(os.path.join(ROOT, "oracle", hdr)).read())
    so = os.path.join(d, "liboracle.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-D_GNU_SOURCE", "-shared", "-fPIC", "-o", so, c,
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
            res = list(ex.map(lambda kv: _run(kv[0], kv[1][0], kv[1][1], tmp), MUTANTS.items()))
    survivors = [n for n, rc in res if rc == 0]
    assert not survivors, f"mistakes no pin caught: {survivors}"
