"""Places synthetic inputs (synth.MoEInputs) in device memory for the C ABI.

Pure data movement: host arrays are copied to the GPU and each expert matrix
is assembled there from the generator's row pool with index_select, giving
the standard layouts of include/moe.h ([E, N, K/2] packed, [E, N, K/32|K/16]
scales, [E] globals); FP4 matrices are then put into the GEMMs' load order
with moe_pack_fp4 (a permutation of bytes).  Nothing here computes a step of
the layer.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import synth
from .moe import (MOE_FMT_BF16, MOE_FMT_FP8S, MOE_FMT_NONE, Layer, Weights, pack_fp4)


def _t(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def pooled_on(pe: synth.PooledExperts, device) -> Weights:
    pool = _t(pe.pool_packed, device)
    pool_s = _t(pe.pool_scales, device)
    idx = torch.from_numpy(pe.idx.astype(np.int64).reshape(-1)).to(device)
    packed = pool.index_select(0, idx).reshape(pe.E, pe.N, -1).contiguous()
    scales = pool_s.index_select(0, idx).reshape(pe.E, pe.N, -1).contiguous()
    g = _t(pe.gscale.astype(np.float32), device)
    return pack_fp4(Weights(pe.fmt, packed, scales, g))


def matrix_on(m: Optional[synth.Matrix], device) -> Weights:
    if m is None:
        return Weights(MOE_FMT_NONE)
    if m.fmt == synth.BF16:
        return Weights(MOE_FMT_BF16, _t(m.bf16, device))
    g = torch.tensor([m.gscale], dtype=torch.float32, device=device)
    if m.fmt == synth.FP8S:  # E4M3 codes [1, N, K] and the weight scale
        return Weights(MOE_FMT_FP8S, _t(m.packed, device)[None], None, g)
    w = Weights(m.fmt, _t(m.packed, device)[None], _t(m.scales, device)[None], g)
    return pack_fp4(w)


def clone_weights(w: Weights) -> Weights:
    c = lambda t: None if t is None else t.clone()
    return Weights(w.fmt, c(w.w), c(w.scales), c(w.global_scale), packed=w.packed)


@dataclass
class DeviceInputs:
    shape: synth.Shape
    x: torch.Tensor
    Wr: torch.Tensor
    bias: Optional[torch.Tensor]
    gamma: torch.Tensor
    w13: Weights
    w2: Weights
    sh13: Weights
    sh2: Weights
    # NVFP4 activations: the input's global (host) and the h globals (device)
    x_global: float = 0.0
    h_globals: Optional[torch.Tensor] = None     # fp32 [E]
    sh_h_global: Optional[torch.Tensor] = None   # fp32 [1]
    # static-FP8 shared expert: the static input scales of its gate/up and down
    sh_in_scale: float = 0.0
    sh_h_scale: float = 0.0

    def layer(self) -> Layer:
        s = self.shape
        return Layer(s.M, s.H, s.E, s.k, s.I, s.I_sh, s.routed_scale, s.eps, self.Wr, self.bias,
                     self.w13, self.w2, self.sh13, self.sh2, self.gamma, s.swiglu_limit,
                     s.act_fmt, self.x_global, self.h_globals,
                     self.sh_h_global if s.sfmt == synth.NVFP4 else None, self.sh_in_scale, self.sh_h_scale)

    def weight_bytes_per_expert(self) -> int:
        s = self.shape
        per = lambda w: (w.w[0].numel() + w.scales.numel() // w.w.shape[0]
                         + (4 if w.global_scale is not None and s.wfmt == synth.NVFP4 else 0))
        return per(self.w13) + per(self.w2)


def to_device(inp: synth.MoEInputs, device="cuda") -> DeviceInputs:
    return DeviceInputs(
        inp.shape,
        _t(inp.x, device),
        _t(inp.Wr, device),
        None if inp.bias is None else _t(inp.bias, device),
        _t(inp.gamma, device),
        pooled_on(inp.w13, device),
        pooled_on(inp.w2, device),
        matrix_on(inp.sh13, device),
        matrix_on(inp.sh2, device),
        float(inp.x_gscale),
        None if inp.h_gscale is None else _t(np.ascontiguousarray(inp.h_gscale, np.float32), device),
        None if inp.h_gscale is None else _t(np.array([inp.sh_h_gscale], np.float32), device),
        float(inp.sh_in13),
        float(inp.sh_in2),
    )
