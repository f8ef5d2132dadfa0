"""Seeded synthetic inputs for the small-M block-scaled-FP4 MoE layer.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only *draws* inputs; it computes no step of the layer (no
routing, no activation quantization, no GEMM, no finalize).  Weights are
handed to the layer already packed, so the offline weight encoders below are
input preparation: the layer never encodes E2M1 or NVFP4 block scales, and
neither the oracle nor the HIP kernels import or call these encoders.

Workloads follow the shapes the pages serve:
  * SGLang-NVIDIA-Mega README, "Supported Models" table and the
    DeepSeek-V4.1 slot table (verify steps of 1-384 rows, 8-row MoE tiles);
  * sgl-nvidia-mega PR #24 (GLM-5.3 NVFP4 spec: one expert group, sigmoid
    scores, renormalized top-8; NVFP4 routed experts with a BF16 shared expert);
  * SGLang Spark GB10 Optimizations, section 1 (NVFP4 K-groups of 16 with FP8
    scale rows and a per-tensor scale).

Recipe (numpy ``Generator(PCG64(seed))``, fixed draw order):
  1. router weight W_r ~ N(0, 1/sqrt(H)), fp32 [E, H];
  2. router bias (workload dependent: none, N(0, 0.01), or Zipf(s) over a
     seeded permutation of expert ranks);
  3. hidden rows x ~ N(0, 1) -> bf16 (truncation of the fp32 draw);
  4. RMSNorm gamma ~ N(1, 0.1) -> bf16 (truncation);
  5. a pool of routed gate_up rows and a pool of routed down rows, each row
     ~ N(0, 0.02) and encoded offline to the workload's FP4 format;
  6. per-expert row index tables into those pools (uniform with replacement);
  7. the shared expert, drawn whole (not pooled).

Pooling keeps every expert matrix a matrix of i.i.d. quantized N(0, 0.02)
rows while drawing only ~8K rows per projection instead of E*2I; each expert
still lives at its own address, so the layer streams E distinct matrices.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Weight / shared-expert formats (match the C ABI's enum values).
MXFP4 = 1
NVFP4 = 2
BF16 = 3
FP8S = 4   # static per-tensor FP8: E4M3 weights, one fp32 weight scale, static input scales (shared expert)
NONE = 0

FMT_NAMES = {NONE: "none", MXFP4: "mxfp4", NVFP4: "nvfp4", BF16: "bf16", FP8S: "fp8s"}
# activation formats of the expert GEMMs
ACT_MXFP8 = 0
ACT_NVFP4 = 1


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)

POOL_ROWS = 8192

# --- format value grids used only by the offline weight encoders -----------
# E2M1 magnitudes indexed by the 3 low bits of a code (OCP MX v1.0 FP4).
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e4m3_positive_grid() -> np.ndarray:
    """Magnitudes of E4M3 codes 0x00..0x7E (0x7F is NaN)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_E4M3_POS = _e4m3_positive_grid()


def _nearest_code(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value (grid ascending); saturates at the top."""
    mids = (grid[1:] + grid[:-1]) * 0.5
    return np.searchsorted(mids, mag, side="left").astype(np.uint8)


def _bf16_trunc(a: np.ndarray) -> np.ndarray:
    """fp32 draws -> bf16 bit patterns by truncation (input preparation only)."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K/2] bytes, low nibble = even K index."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def encode_mxfp4_rows(w: np.ndarray):
    """Offline MXFP4 encoding of fp32 rows [N, K] (K % 32 == 0).

    Block scale 2^(floor(log2 amax) - 2), E2M1 elements nearest, saturating.
    Returns (packed [N, K/2] u8, scales [N, K/32] u8 E8M0 codes)."""
    n, k = w.shape
    blk = w.reshape(n, k // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int32)
    v = blk * np.ldexp(1.0, -e)[..., None]
    codes = _nearest_code(np.abs(v), _E2M1_MAG) | (np.signbit(v).astype(np.uint8) << 3)
    return _pack_nibbles(codes.reshape(n, k)), (e + 127).astype(np.uint8)


def encode_nvfp4_rows(w: np.ndarray, global_scale: float):
    """Offline NVFP4 encoding of fp32 rows [N, K] (K % 16 == 0) with a given
    per-tensor fp32 global scale: E4M3 block scale per 16 (nearest of
    amax/(6*global)), E2M1 elements nearest, saturating.
    Returns (packed [N, K/2] u8, scales [N, K/16] u8 E4M3 codes)."""
    n, k = w.shape
    blk = w.reshape(n, k // 16, 16).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    sc = _nearest_code(amax / (6.0 * global_scale), _E4M3_POS)
    sval = _E4M3_POS[sc] * global_scale
    v = blk / np.where(sval > 0, sval, 1.0)[..., None]
    v = np.where((sval > 0)[..., None], v, 0.0)
    codes = _nearest_code(np.abs(v), _E2M1_MAG) | (np.signbit(v).astype(np.uint8) << 3)
    return _pack_nibbles(codes.reshape(n, k)), sc.astype(np.uint8)


def nvfp4_global_for(w: np.ndarray) -> np.float32:
    """ModelOpt-style per-tensor scale amax / (6 * 448) as fp32."""
    return np.float32(max(float(np.abs(w).max()), 1e-30) / (6.0 * 448.0))


# --- workloads -------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    name: str
    M: int
    H: int
    E: int
    k: int
    I: int
    wfmt: int
    sfmt: int
    I_sh: int
    routed_scale: float
    bias: str  # "none" | "normal:<std>" | "zipf:<s>"
    eps: float = 1e-6
    desc: str = ""
    swiglu_limit: float = 0.0  # clamped SwiGLU of every expert; 0: unclamped
    act_fmt: int = 0           # ACT_MXFP8, or ACT_NVFP4 (W4A4: NVFP4 experts only)


# The five workloads the layer is measured on (pages: DeepSeek-V4.1 verify
# widths, GLM-5.3 NVFP4 verify with sigmoid top-8, Kimi K3 packed MXFP4 decode).
WORKLOADS = {
    "tiny-m4-h1024-e16-k4-mxfp4": Shape(
        "tiny-m4-h1024-e16-k4-mxfp4", 4, 1024, 16, 4, 512, MXFP4, NONE, 0, 1.0, "normal:0.01",
        desc="tiny layer: 4 rows, MXFP4 experts, router bias N(0,0.01), no shared expert"),
    "verify-m8-h7168-e256-k8-nvfp4": Shape(
        "verify-m8-h7168-e256-k8-nvfp4", 8, 7168, 256, 8, 256, NVFP4, BF16, 256, 2.5, "none",
        desc="verify step, 2 requests x 4 draft tokens; one GPU's TP8 share (I=2048/8); "
             "NVFP4 experts, bf16 shared expert, routed scale 2.5"),
    "decode-m16-h7168-e384-k8-mxfp4": Shape(
        "decode-m16-h7168-e384-k8-mxfp4", 16, 7168, 384, 8, 2048, MXFP4, MXFP4, 2048, 1.0, "none",
        desc="one-token decode at 16 rows; one GPU holding an expert-parallel slice; "
             "packed MXFP4 experts and MXFP4 shared expert"),
    "skew-m48-h4096-e512-k10-nvfp4": Shape(
        "skew-m48-h4096-e512-k10-nvfp4", 48, 4096, 512, 10, 512, NVFP4, BF16, 512, 1.0, "zipf:1.2",
        desc="skewed routing at 48 rows: Zipf(1.2) router bias so several experts take "
             "more than one 8-row tile; NVFP4 experts, bf16 shared expert"),
    "wide-m384-h7168-e256-k8-mxfp4": Shape(
        "wide-m384-h7168-e256-k8-mxfp4", 384, 7168, 256, 8, 2048, MXFP4, MXFP4, 2048, 1.0, "none",
        desc="wide verify step, 64 requests x 6 draft tokens; MXFP4 experts, MXFP4 shared expert"),
}
WORKLOAD_ORDER = list(WORKLOADS)

# Further workloads (not among the five): NVFP4 activations (W4A4) at the
# pages' Qwen3.5 verify step of 7 rows with top-10 (README slot table, rows
# "route" and "mkm"), with the static-FP8 shared expert of the same table
# (row "route_shared"); the pages give no layer dimensions, so it takes the
# skewed-routing workload's (hidden 4096, 512 experts, intermediate 512,
# shared expert of 512) without the bias.
EXTRA_WORKLOADS = {
    "verify7-m7-h4096-e512-k10-nvfp4-a4": Shape(
        "verify7-m7-h4096-e512-k10-nvfp4-a4", 7, 4096, 512, 10, 512, NVFP4, FP8S, 512, 1.0, "none",
        act_fmt=ACT_NVFP4,
        desc="7-row verify step with top-10, NVFP4 experts on NVFP4 activations (W4A4), static-FP8 shared expert"),
}
WORKLOADS.update(EXTRA_WORKLOADS)


def seed_of(name: str) -> int:
    """Default seed of a named workload: 1-5 for the five, 101.. for the others."""
    if name in WORKLOAD_ORDER:
        return WORKLOAD_ORDER.index(name) + 1
    return 101 + list(EXTRA_WORKLOADS).index(name)


def custom_shape(M, H, E, k, I, wfmt=MXFP4, sfmt=NONE, I_sh=None, routed_scale=1.0,
                 bias="none", eps=1e-6, name=None, swiglu_limit=0.0, act_fmt=0) -> Shape:
    I_sh = I if I_sh is None else I_sh
    if sfmt == NONE:
        I_sh = 0
    name = name or f"custom-m{M}-h{H}-e{E}-k{k}-i{I}-{FMT_NAMES[wfmt]}-sh{FMT_NAMES[sfmt]}"
    if swiglu_limit:
        name += f"-clamp{swiglu_limit:g}"
    if act_fmt == ACT_NVFP4:
        name += "-a4"
    return Shape(name, M, H, E, k, I, wfmt, sfmt, I_sh, float(routed_scale), bias, eps,
                 swiglu_limit=float(swiglu_limit), act_fmt=int(act_fmt))


@dataclass
class Matrix:
    """One weight matrix [N, K] in the layer's canonical layout.

    fmt MXFP4/NVFP4: ``packed`` [N, K/2] u8 (low nibble = even K), ``scales``
    [N, K/32] E8M0 (MX) or [N, K/16] E4M3 (NV), ``gscale`` fp32 (NV only).
    fmt BF16: ``bf16`` [N, K] u16.
    fmt FP8S: ``packed`` [N, K] E4M3 codes, ``gscale`` the fp32 weight scale."""
    fmt: int
    N: int
    K: int
    packed: Optional[np.ndarray] = None
    scales: Optional[np.ndarray] = None
    gscale: float = 1.0
    bf16: Optional[np.ndarray] = None


@dataclass
class PooledExperts:
    """E expert matrices [N, K] assembled from a pool: expert e, row n is pool
    row ``idx[e, n]``.  ``gscale[e]`` is the per-expert fp32 global (NV)."""
    fmt: int
    E: int
    N: int
    K: int
    pool_packed: np.ndarray
    pool_scales: np.ndarray
    idx: np.ndarray
    gscale: np.ndarray

    def expert(self, e: int) -> Matrix:
        rows = self.idx[e]
        return Matrix(self.fmt, self.N, self.K, np.ascontiguousarray(self.pool_packed[rows]),
                      np.ascontiguousarray(self.pool_scales[rows]), float(self.gscale[e]))

    def full_packed(self) -> np.ndarray:
        return np.ascontiguousarray(self.pool_packed[self.idx])

    def full_scales(self) -> np.ndarray:
        return np.ascontiguousarray(self.pool_scales[self.idx])


@dataclass
class MoEInputs:
    shape: Shape
    seed: int
    x: np.ndarray            # bf16 bits [M, H]; also the residual (out = RMSNorm(x + MoE(x)))
    Wr: np.ndarray           # fp32 [E, H]
    bias: Optional[np.ndarray]  # fp32 [E] or None
    gamma: np.ndarray        # bf16 bits [H]
    w13: PooledExperts       # [E, 2I, H]
    w2: PooledExperts        # [E, H, I]
    sh13: Optional[Matrix] = None  # [2I_sh, H]
    sh2: Optional[Matrix] = None   # [H, I_sh]
    meta: dict = field(default_factory=dict)
    # NVFP4 activations (act_fmt ACT_NVFP4): static globals of the layer input,
    # of each routed expert's h and of the shared expert's h
    x_gscale: float = 0.0
    h_gscale: Optional[np.ndarray] = None  # fp32 [E]
    sh_h_gscale: float = 0.0
    # static-FP8 shared expert (sfmt FP8S): static input scales of its gate/up
    # (the layer input) and of its down (h)
    sh_in13: float = 0.0
    sh_in2: float = 0.0

    @property
    def residual(self) -> np.ndarray:
        return self.x


def _draw_bias(rng, shape: Shape):
    kind = shape.bias
    if kind == "none":
        return None
    if kind.startswith("normal:"):
        std = float(kind.split(":")[1])
        return (rng.standard_normal(shape.E) * std).astype(np.float32)
    if kind.startswith("zipf:"):
        s = float(kind.split(":")[1])
        rank = rng.permutation(shape.E) + 1
        return (rank.astype(np.float64) ** (-s)).astype(np.float32)
    raise ValueError(f"unknown bias kind {kind!r}")


def _encode(fmt, w, gscale=None):
    if fmt == MXFP4:
        return encode_mxfp4_rows(w)
    if fmt == NVFP4:
        return encode_nvfp4_rows(w, float(gscale))
    raise ValueError(fmt)


def _pooled(rng, fmt, E, N, K, pool_rows, std=0.02) -> PooledExperts:
    r = int(min(pool_rows, E * N))
    w = (rng.standard_normal((r, K), dtype=np.float32) * np.float32(std))
    g = nvfp4_global_for(w) if fmt == NVFP4 else np.float32(1.0)
    packed, scales = _encode(fmt, w, g)
    idx = rng.integers(0, r, size=(E, N), dtype=np.int64).astype(np.int32)
    return PooledExperts(fmt, E, N, K, packed, scales, idx, np.full(E, g, dtype=np.float32))


def encode_fp8s(w: np.ndarray):
    """Offline static-FP8 encoding of an fp32 matrix: one per-tensor scale
    amax / 448 (fp32) and E4M3 elements nearest, saturating.
    Returns (codes [N, K] u8, scale)."""
    s = np.float32(max(float(np.abs(w).max()), 1e-30) / 448.0)
    v = w.astype(np.float64) / np.float64(s)
    codes = _nearest_code(np.abs(v), _E4M3_POS) | (np.signbit(v).astype(np.uint8) << 7)
    return codes.astype(np.uint8), float(s)


def _whole(rng, fmt, N, K, std=0.02) -> Matrix:
    w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(std))
    if fmt == BF16:
        return Matrix(BF16, N, K, bf16=_bf16_trunc(w))
    if fmt == FP8S:
        codes, sc = encode_fp8s(w)
        return Matrix(FP8S, N, K, packed=codes, gscale=sc)
    g = nvfp4_global_for(w) if fmt == NVFP4 else np.float32(1.0)
    packed, scales = _encode(fmt, w, g)
    return Matrix(fmt, N, K, packed, scales, float(g))


def make_inputs(shape: Shape | str, seed: int = 1, pool_rows: int = POOL_ROWS) -> MoEInputs:
    """Draw every input of one layer step (see the module docstring)."""
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    rng = np.random.Generator(np.random.PCG64(seed))
    M, H, E, I = shape.M, shape.H, shape.E, shape.I
    Wr = (rng.standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H)))
    bias = _draw_bias(rng, shape)
    x = _bf16_trunc(rng.standard_normal((M, H), dtype=np.float32))
    gamma = _bf16_trunc(1.0 + 0.1 * rng.standard_normal(H, dtype=np.float32))
    w13 = _pooled(rng, shape.wfmt, E, 2 * I, H, pool_rows)
    w2 = _pooled(rng, shape.wfmt, E, H, I, pool_rows)
    sh13 = sh2 = None
    if shape.sfmt != NONE:
        sh13 = _whole(rng, shape.sfmt, 2 * shape.I_sh, H)
        sh2 = _whole(rng, shape.sfmt, H, shape.I_sh)
    inp = MoEInputs(shape, seed, x, Wr, bias, gamma, w13, w2, sh13, sh2)
    if shape.sfmt == FP8S:
        # Static input scales, as an FP8 checkpoint ships them (calibrated
        # offline; no draw): the gate/up input's from this step's amax, the
        # down input's from 16x the spread of h (gate and up each have a std
        # of 0.02 sqrt(H) for N(0, 1) rows and N(0, 0.02) weights), so only
        # rare outliers of h saturate.
        xa = np.abs(bf16_to_f32(x)).max()
        inp.sh_in13 = float(np.float32(xa) / np.float32(448))
        inp.sh_in2 = float(np.float32(16.0 * (0.02 * np.sqrt(H)) ** 2) / np.float32(448))
    if shape.act_fmt == ACT_NVFP4:
        if shape.wfmt != NVFP4 or shape.sfmt == MXFP4:
            raise ValueError("NVFP4 activations go with NVFP4 experts (shared: none, NVFP4, bf16 or FP8S)")
        # Static globals, as an NVFP4 checkpoint ships them (calibrated offline):
        # the input's from this step's own amax; each h's from the spread that
        # gate and up have for N(0, 1) rows and N(0, 0.02) weights (std
        # 0.02 sqrt(H) each, so h = silu(g) u spreads about their product),
        # times 2^u, u in {-1, 0, 1} per expert.  Drawn after everything else, so
        # the other inputs of a seed do not change.
        xa = np.abs(bf16_to_f32(x)).max()
        inp.x_gscale = float(np.float32(xa) / np.float32(6 * 448))
        var = np.float32((0.02 * np.sqrt(H)) ** 2)
        base = np.float32(8.0) * var / np.float32(6 * 448)
        inp.h_gscale = (base * np.exp2(rng.integers(-1, 2, size=E)).astype(np.float32)).astype(np.float32)
        inp.sh_h_gscale = float(base)
    return inp


def vary_globals(inp: MoEInputs, seed: int) -> MoEInputs:
    """Give every NVFP4 expert its own global scale (x 2^u, u in {-1,0,1}), so
    per-expert globals are exercised; the weights stay exactly representable."""
    if inp.shape.wfmt != NVFP4:
        return inp
    rng = np.random.Generator(np.random.PCG64(seed))
    for pe in (inp.w13, inp.w2):
        pe.gscale = (pe.gscale * np.exp2(rng.integers(-1, 2, size=pe.E))).astype(np.float32)
    return inp
