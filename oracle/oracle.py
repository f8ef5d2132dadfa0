"""ctypes front-end of the reference CPU implementation (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the package's smoke
check and by the benchmark's CPU-baseline leg.  The layer's product path never
imports this module.  See moe_oracle.h for what each function computes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB lets the mutation tests point the pins at a deliberately
# broken copy of the oracle.
LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "moe_oracle.c")]

ORC_NONE, ORC_MXFP4, ORC_NVFP4, ORC_BF16, ORC_FP8S = 0, 1, 2, 3, 4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-shared", "-fPIC",
               "-o", tmp] + SOURCES + ["-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class orc_mat(C.Structure):
    _fields_ = [("fmt", C.c_int), ("packed", C.c_void_p), ("scales", C.c_void_p),
                ("gscale", C.c_float), ("bf16", C.c_void_p)]


class orc_layer(C.Structure):
    _fields_ = [("M", C.c_int), ("H", C.c_int), ("E", C.c_int), ("k", C.c_int),
                ("I", C.c_int), ("I_sh", C.c_int), ("wfmt", C.c_int), ("sfmt", C.c_int),
                ("routed_scale", C.c_double), ("eps", C.c_double),
                ("x", C.c_void_p), ("residual", C.c_void_p), ("gamma", C.c_void_p),
                ("Wr", C.c_void_p), ("bias", C.c_void_p),
                ("w13", C.POINTER(orc_mat)), ("w2", C.POINTER(orc_mat)),
                ("sh13", orc_mat), ("sh2", orc_mat), ("swiglu_limit", C.c_double),
                ("act_fmt", C.c_int), ("x_gscale", C.c_float), ("h_gscale", C.c_void_p),
                ("sh_h_gscale", C.c_float), ("sh_in13", C.c_float), ("sh_in2", C.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = C.CDLL(LIB_PATH)
        d, u8, i32, f32 = C.c_double, C.c_uint8, C.c_int32, C.c_float
        vp = C.c_void_p
        L.orc_e2m1_value.restype = d
        L.orc_e4m3_value.restype = d
        L.orc_e8m0_value.restype = d
        L.orc_bf16_value.restype = d
        L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_bf16_rne.restype = C.c_uint16
        L.orc_bf16_rne.argtypes = [d]
        L.orc_e4m3_rne_sat.restype = u8
        L.orc_e4m3_rne_sat.argtypes = [d]
        L.orc_mxfp8_quant_block.argtypes = [vp, vp, vp]
        L.orc_e4m3_rne_sat_n.argtypes = [vp, C.c_int, vp]
        L.orc_bf16_rne_n.argtypes = [vp, C.c_int, vp]
        L.orc_mxfp8_quant_bf16.argtypes = [vp, C.c_int, C.c_int, vp, vp]
        L.orc_mxfp8_quant_f64.argtypes = [vp, C.c_int, C.c_int, vp, vp]
        L.orc_mxfp8_dequant.argtypes = [vp, vp, C.c_int, vp]
        L.orc_e2m1_rne_sat.restype = u8
        L.orc_e2m1_rne_sat.argtypes = [f32]
        L.orc_nvfp4_quant_block.argtypes = [vp, f32, vp, vp]
        L.orc_nvfp4_quant_f32.argtypes = [vp, C.c_int, C.c_int, f32, vp, vp]
        L.orc_nvfp4_quant_bf16.argtypes = [vp, C.c_int, C.c_int, f32, vp, vp]
        L.orc_nvfp4_dequant.argtypes = [vp, vp, C.c_int, f32, vp]
        L.orc_mat_row.argtypes = [C.POINTER(orc_mat), C.c_int, C.c_int, vp]
        L.orc_router_logits.argtypes = [vp, vp, C.c_int, C.c_int, C.c_int, vp]
        L.orc_topk_row.argtypes = [vp, vp, C.c_int, C.c_int, d, vp, vp, vp]
        L.orc_route.argtypes = [vp, vp, C.c_int, C.c_int, C.c_int, d] + [vp] * 8
        L.orc_gate_up.argtypes = [C.POINTER(orc_mat), C.c_int, C.c_int, vp, d, vp]
        L.orc_gate_up_bf16.argtypes = [C.POINTER(orc_mat), C.c_int, C.c_int, vp, d, vp]
        L.orc_swiglu.restype = d
        L.orc_swiglu.argtypes = [d, d, d]
        L.orc_down.argtypes = [C.POINTER(orc_mat), C.c_int, C.c_int, vp, vp]
        L.orc_fp8s_quant.restype = u8
        L.orc_fp8s_quant.argtypes = [f32, f32]
        L.orc_gate_up_fp8s.argtypes = [C.POINTER(orc_mat), C.c_int, C.c_int, vp, f32, d, vp, vp]
        L.orc_down_fp8s.argtypes = [C.POINTER(orc_mat), C.c_int, C.c_int, vp, f32, vp, vp]
        L.orc_finalize_row.argtypes = [C.c_int, C.c_int, vp, vp, vp, vp, vp, d, vp, vp, vp]
        L.orc_moe_rows.argtypes = [C.POINTER(orc_layer), vp, vp, C.c_int, C.c_int] + [vp] * 9
        L.orc_moe_rows.restype = C.c_int
        L.orc_num_cores.restype = C.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


# ---- formats ---------------------------------------------------------------

def e2m1_table() -> np.ndarray:
    return np.array([lib().orc_e2m1_value(c) for c in range(16)])


def e4m3_table() -> np.ndarray:
    return np.array([lib().orc_e4m3_value(c) for c in range(256)])


def e8m0_table() -> np.ndarray:
    return np.array([lib().orc_e8m0_value(c) for c in range(256)])


def bf16_value(bits) -> float:
    return lib().orc_bf16_value(int(bits))


def bf16_rne(v: float) -> int:
    return int(lib().orc_bf16_rne(float(v)))


def e4m3_rne_sat(v: float) -> int:
    return int(lib().orc_e4m3_rne_sat(float(v)))


def e4m3_rne_sat_n(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64).ravel()
    out = np.empty(v.shape[0], np.uint8)
    lib().orc_e4m3_rne_sat_n(_p(v), v.shape[0], _p(out))
    return out


def bf16_rne_n(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float64).ravel()
    out = np.empty(v.shape[0], np.uint16)
    lib().orc_bf16_rne_n(_p(v), v.shape[0], _p(out))
    return out


def mxfp8_quant_f64(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.float64)
    M, K = v.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 32), np.uint8)
    lib().orc_mxfp8_quant_f64(_p(v), M, K, _p(q), _p(s))
    return q, s


def mxfp8_quant_bf16(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = x.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 32), np.uint8)
    lib().orc_mxfp8_quant_bf16(_p(x), M, K, _p(q), _p(s))
    return q, s


def e2m1_rne_sat(v: float) -> int:
    return int(lib().orc_e2m1_rne_sat(float(v)))


def nvfp4_quant_f32(v: np.ndarray, g: float):
    """NVFP4 activation quant of fp32 rows [M, K] with global g: codes [M, K/2]
    (even element in the low nibble), E4M3 scales [M, K/16]."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    M, K = v.shape
    q = np.empty((M, K // 2), np.uint8)
    s = np.empty((M, K // 16), np.uint8)
    lib().orc_nvfp4_quant_f32(_p(v), M, K, float(g), _p(q), _p(s))
    return q, s


def nvfp4_quant_bf16(x: np.ndarray, g: float):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = x.shape
    q = np.empty((M, K // 2), np.uint8)
    s = np.empty((M, K // 16), np.uint8)
    lib().orc_nvfp4_quant_bf16(_p(x), M, K, float(g), _p(q), _p(s))
    return q, s


def nvfp4_dequant(q: np.ndarray, s: np.ndarray, g: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    M, K = q.shape[0], 2 * q.shape[1]
    out = np.empty((M, K), np.float64)
    for r in range(M):
        lib().orc_nvfp4_dequant(_p(q[r]), _p(s[r]), K, float(g), _p(out[r]))
    return out


def mxfp8_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    M, K = q.shape
    out = np.empty((M, K), np.float64)
    for r in range(M):
        lib().orc_mxfp8_dequant(_p(q[r]), _p(s[r]), K, _p(out[r]))
    return out


# ---- matrices --------------------------------------------------------------

class Mat:
    """Keeps the numpy buffers of one orc_mat alive."""

    def __init__(self, fmt, packed=None, scales=None, gscale=1.0, bf16=None):
        self.fmt = fmt
        self.packed = None if packed is None else np.ascontiguousarray(packed, np.uint8)
        self.scales = None if scales is None else np.ascontiguousarray(scales, np.uint8)
        self.bf16 = None if bf16 is None else np.ascontiguousarray(bf16, np.uint16)
        self.gscale = float(gscale)

    @classmethod
    def from_synth(cls, m):
        if m is None:
            return cls(ORC_NONE)
        return cls(m.fmt, m.packed, m.scales, m.gscale, m.bf16)

    def c(self) -> orc_mat:
        return orc_mat(self.fmt, _p(self.packed), _p(self.scales), self.gscale, _p(self.bf16))


def mat_dequant(m: Mat, N: int, K: int) -> np.ndarray:
    out = np.empty((N, K), np.float64)
    cm = m.c()
    for n in range(N):
        lib().orc_mat_row(C.byref(cm), K, n, _p(out[n]))
    return out


# ---- router ----------------------------------------------------------------

def router_logits(x, Wr) -> np.ndarray:
    x = np.ascontiguousarray(x, np.uint16)
    Wr = np.ascontiguousarray(Wr, np.float32)
    M, H = x.shape
    E = Wr.shape[0]
    out = np.empty((M, E), np.float64)
    lib().orc_router_logits(_p(x), _p(Wr), M, H, E, _p(out))
    return out


def route(logits: np.ndarray, bias, k: int, scale: float):
    logits = np.ascontiguousarray(logits, np.float32)
    M, E = logits.shape
    P = M * k
    tmax = tile_capacity(M, E, k)
    ids = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float32)
    offsets = np.empty(E + 1, np.int32)
    bucket = np.empty(max(P, 1), np.int32)
    te = np.full(max(tmax, 1), -1, np.int32)
    tb = np.full(max(tmax, 1), -1, np.int32)
    tr = np.full(max(tmax, 1), -1, np.int32)
    nt = np.zeros(1, np.int32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().orc_route(_p(logits), _p(b), M, E, k, float(scale), _p(ids), _p(w), _p(offsets),
                    _p(bucket), _p(te), _p(tb), _p(tr), _p(nt))
    n = int(nt[0])
    return dict(ids=ids, w=w, offsets=offsets, bucket=bucket[:P], tile_expert=te[:n],
                tile_begin=tb[:n], tile_rows=tr[:n], num_tiles=n)


def tile_capacity(M: int, E: int, k: int) -> int:
    """Upper bound on the 8-row tile count: sum ceil(n_e/8) <= P/8 + min(E, P)."""
    P = M * k
    return (P + 7) // 8 + min(E, P)


def topk_row(logits_row, bias, k, scale):
    lr = np.ascontiguousarray(logits_row, np.float32)
    E = lr.shape[0]
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float32)
    s = np.empty(k, np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().orc_topk_row(_p(lr), _p(b), E, k, float(scale), _p(ids), _p(w), _p(s))
    return ids, w, s


# ---- experts / finalize ----------------------------------------------------

def swiglu(g: float, u: float, limit: float = 0.0) -> float:
    return float(lib().orc_swiglu(float(g), float(u), float(limit)))


def gate_up(m: Mat, H: int, I: int, a: np.ndarray, limit: float = 0.0) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float64)
    h = np.empty(I, np.float64)
    cm = m.c()
    lib().orc_gate_up(C.byref(cm), H, I, _p(a), float(limit), _p(h))
    return h


def gate_up_bf16(m: Mat, H: int, I: int, x_row: np.ndarray, limit: float = 0.0) -> np.ndarray:
    x_row = np.ascontiguousarray(x_row, np.uint16)
    h = np.empty(I, np.float64)
    cm = m.c()
    lib().orc_gate_up_bf16(C.byref(cm), H, I, _p(x_row), float(limit), _p(h))
    return h


def down(m: Mat, H: int, I: int, h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.float64)
    y = np.empty(H, np.float64)
    cm = m.c()
    lib().orc_down(C.byref(cm), H, I, _p(h), _p(y))
    return y


def fp8s_quant(v: float, s_in: float) -> int:
    """Static-FP8 code of one value: E4M3 of the fp32 quotient v / s_in."""
    return int(lib().orc_fp8s_quant(float(v), float(s_in)))


def gate_up_fp8s(m: Mat, H: int, I: int, x_row: np.ndarray, s_in: float, limit: float = 0.0):
    """Static-FP8 shared gate/up on one bf16 row: (h bf16 bits [I], g/u bf16 bits [2I])."""
    x_row = np.ascontiguousarray(x_row, np.uint16)
    h = np.empty(I, np.uint16)
    gu = np.empty(2 * I, np.uint16)
    cm = m.c()
    lib().orc_gate_up_fp8s(C.byref(cm), H, I, _p(x_row), float(s_in), float(limit), _p(h), _p(gu))
    return h, gu


def down_fp8s(m: Mat, H: int, I: int, h_bf16: np.ndarray, s_in: float):
    """Static-FP8 shared down on bf16 h: (y fp64 [H], h codes [I])."""
    h_bf16 = np.ascontiguousarray(h_bf16, np.uint16)
    y = np.empty(H, np.float64)
    hq = np.empty(I, np.uint8)
    cm = m.c()
    lib().orc_down_fp8s(C.byref(cm), H, I, _p(h_bf16), float(s_in), _p(y), _p(hq))
    return y, hq


def finalize_row(y, w, y_sh, residual, gamma, eps):
    y = np.ascontiguousarray(y, np.float64)
    k, H = y.shape
    w = np.ascontiguousarray(w, np.float32)
    ysh = None if y_sh is None else np.ascontiguousarray(y_sh, np.float64)
    residual = np.ascontiguousarray(residual, np.uint16)
    gamma = np.ascontiguousarray(gamma, np.uint16)
    out64 = np.empty(H, np.float64)
    ob = np.empty(H, np.uint16)
    ro = np.empty(H, np.uint16)
    lib().orc_finalize_row(H, k, _p(y), _p(w), _p(ysh), _p(residual), _p(gamma), float(eps),
                           _p(out64), _p(ob), _p(ro))
    return out64, ob, ro


# ---- the layer ---------------------------------------------------------------

class Layer:
    """An orc_layer over synthetic inputs; only the experts in ``experts`` (or
    all of them) get decoded weight pointers, the rest stay null."""

    def __init__(self, inp, experts: Optional[Sequence[int]] = None, w13_full=None, w2_full=None):
        sh = inp.shape
        self.inp = inp
        E = sh.E
        self.mats13 = [None] * E
        self.mats2 = [None] * E
        ex = range(E) if experts is None else sorted(set(int(e) for e in experts))
        for e in ex:
            m13 = inp.w13.expert(e)
            m2 = inp.w2.expert(e)
            self.mats13[e] = Mat(m13.fmt, m13.packed, m13.scales, m13.gscale)
            self.mats2[e] = Mat(m2.fmt, m2.packed, m2.scales, m2.gscale)
        none = Mat(ORC_NONE)
        arr13 = (orc_mat * E)(*[(m or none).c() for m in self.mats13])
        arr2 = (orc_mat * E)(*[(m or none).c() for m in self.mats2])
        self._arr13, self._arr2 = arr13, arr2
        self.sh13 = Mat.from_synth(inp.sh13)
        self.sh2 = Mat.from_synth(inp.sh2)
        self.x = np.ascontiguousarray(inp.x, np.uint16)
        self.gamma = np.ascontiguousarray(inp.gamma, np.uint16)
        self.Wr = np.ascontiguousarray(inp.Wr, np.float32)
        self.bias = None if inp.bias is None else np.ascontiguousarray(inp.bias, np.float32)
        self.h_g = None if inp.h_gscale is None else np.ascontiguousarray(inp.h_gscale, np.float32)
        self.c = orc_layer(sh.M, sh.H, sh.E, sh.k, sh.I, sh.I_sh, sh.wfmt, sh.sfmt,
                           float(sh.routed_scale), float(sh.eps), _p(self.x), _p(self.x),
                           _p(self.gamma), _p(self.Wr), _p(self.bias), arr13, arr2,
                           self.sh13.c(), self.sh2.c(), float(sh.swiglu_limit), int(sh.act_fmt),
                           float(inp.x_gscale), _p(self.h_g), float(inp.sh_h_gscale),
                           float(inp.sh_in13), float(inp.sh_in2))

    def rows(self, rows, logits=None, nthreads=0, want_h=False):
        sh = self.inp.shape
        rows = np.ascontiguousarray(rows, np.int32)
        n = len(rows)
        lg = None if logits is None else np.ascontiguousarray(logits, np.float32)
        out64 = np.empty((n, sh.H), np.float64)
        ob = np.empty((n, sh.H), np.uint16)
        ro = np.empty((n, sh.H), np.uint16)
        ids = np.empty((n, sh.k), np.int32)
        w = np.empty((n, sh.k), np.float32)
        y = np.empty((n, sh.k, sh.H), np.float64)
        ysh = np.zeros((n, sh.H), np.float64)
        a4 = sh.act_fmt == 1
        hq = np.empty((n, sh.k, sh.I // 2 if a4 else sh.I), np.uint8) if want_h else None
        hs = np.empty((n, sh.k, sh.I // 16 if a4 else sh.I // 32), np.uint8) if want_h else None
        rc = lib().orc_moe_rows(C.byref(self.c), _p(lg), _p(rows), n, int(nthreads), _p(out64),
                                _p(ob), _p(ro), _p(ids), _p(w), _p(y), _p(ysh), _p(hq), _p(hs))
        if rc != 0:
            raise ValueError("orc_moe_rows rejected its arguments")
        return dict(out64=out64, out_bf16=ob, resid_out=ro, ids=ids, w=w, y=y, y_sh=ysh,
                    hq=hq, hs=hs)


def num_cores() -> int:
    return int(lib().orc_num_cores())
