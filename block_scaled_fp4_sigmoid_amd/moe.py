"""Python binding of the C ABI in include/moe.h (ctypes; argument marshalling only).

Every step of the layer runs in the HIP library libmoe_mi355.so; this module
only turns torch tensors (device memory) and torch streams into the plain
pointers the C ABI takes.  There is no fallback: if the library is missing or
a call returns an error, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355.so")

MOE_FMT_NONE, MOE_FMT_MXFP4, MOE_FMT_NVFP4, MOE_FMT_BF16, MOE_FMT_FP8S = 0, 1, 2, 3, 4
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_ERR_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ["moe_status_str", "moe_abi_version", "moe_tile_capacity", "moe_packed_scale_bytes",
           "moe_pack_fp4", "moe_route_workspace_bytes",
           "moe_route_topk", "moe_quant_act_mxfp8", "moe_quant_act_nvfp4", "moe_gate_up_workspace_bytes",
           "moe_expert_gate_up", "moe_expert_gate_up_tok", "moe_expert_down", "moe_expert_gate_up_nvfp4a",
           "moe_expert_down_nvfp4a", "moe_finalize_rmsnorm",
           "moe_finalize_rmsnorm_mxfp8", "moe_layer_workspace_bytes", "moe_layer",
           "moe_layer_mxfp8_out", "moe_layer_noalloc", "moe_expert_gate_up_fp8s", "moe_expert_down_fp8s"]


class moe_weights(C.Structure):
    _fields_ = [("fmt", C.c_int), ("w", C.c_void_p), ("scales", C.c_void_p),
                ("global_scale", C.c_void_p)]


class moe_routing(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_ids", "topk_w", "expert_offsets", "bucket",
                                          "tile_expert", "tile_begin", "tile_rows", "num_tiles",
                                          "active_experts", "num_active", "active_offsets")]


class moe_layer_desc(C.Structure):
    _fields_ = [("M", C.c_int), ("H", C.c_int), ("E", C.c_int), ("k", C.c_int), ("I", C.c_int),
                ("I_sh", C.c_int), ("routed_scale", C.c_float), ("eps", C.c_float),
                ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("w13", moe_weights), ("w2", moe_weights), ("sh13", moe_weights),
                ("sh2", moe_weights), ("gamma", C.c_void_p), ("swiglu_limit", C.c_float),
                ("act_fmt", C.c_int), ("x_global", C.c_float), ("h_globals", C.c_void_p),
                ("sh_h_global", C.c_void_p), ("sh_in_scale", C.c_float), ("sh_h_scale", C.c_float)]


_lib = None


def lib() -> C.CDLL:
    """The HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m "
                               "block_scaled_fp4_sigmoid_amd.build or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        vp, i, f, sz = C.c_void_p, C.c_int, C.c_float, C.c_size_t
        L.moe_status_str.restype = C.c_char_p
        L.moe_status_str.argtypes = [i]
        L.moe_abi_version.restype = i
        L.moe_tile_capacity.restype = i
        L.moe_tile_capacity.argtypes = [i, i, i]
        L.moe_packed_scale_bytes.restype = sz
        L.moe_packed_scale_bytes.argtypes = [i, i, i, i]
        L.moe_pack_fp4.restype = i
        L.moe_pack_fp4.argtypes = [i, i, i, i, vp, vp, vp, vp, vp]
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route_workspace_bytes.argtypes = [i, i, i, i]
        L.moe_route_topk.restype = i
        L.moe_route_topk.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp, C.POINTER(moe_routing), vp, sz, vp]
        L.moe_quant_act_mxfp8.restype = i
        L.moe_quant_act_mxfp8.argtypes = [vp, i, i, C.POINTER(moe_routing), i, vp, vp, vp]
        L.moe_quant_act_nvfp4.restype = i
        L.moe_quant_act_nvfp4.argtypes = [vp, i, i, f, C.POINTER(moe_routing), i, vp, vp, vp]
        L.moe_gate_up_workspace_bytes.restype = sz
        L.moe_gate_up_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.moe_expert_gate_up.restype = i
        L.moe_expert_gate_up.argtypes = [C.POINTER(moe_weights), vp, vp, vp, C.POINTER(moe_routing),
                                         i, i, i, i, i, f, vp, vp, vp, vp, sz, vp]
        L.moe_expert_gate_up_tok.restype = i
        L.moe_expert_gate_up_tok.argtypes = [C.POINTER(moe_weights), vp, vp, C.POINTER(moe_routing),
                                             i, i, i, i, i, f, vp, vp, vp, sz, vp]
        L.moe_expert_down.restype = i
        L.moe_expert_down.argtypes = [C.POINTER(moe_weights), vp, vp, vp, C.POINTER(moe_routing),
                                      i, i, i, i, i, vp, vp]
        L.moe_expert_gate_up_nvfp4a.restype = i
        L.moe_expert_gate_up_nvfp4a.argtypes = [C.POINTER(moe_weights), vp, vp, f, C.POINTER(moe_routing),
                                                i, i, i, i, i, f, vp, vp, vp, vp]
        L.moe_expert_down_nvfp4a.restype = i
        L.moe_expert_down_nvfp4a.argtypes = [C.POINTER(moe_weights), vp, vp, vp, C.POINTER(moe_routing),
                                             i, i, i, i, i, vp, vp]
        L.moe_finalize_rmsnorm.restype = i
        L.moe_finalize_rmsnorm.argtypes = [vp, vp, vp, vp, vp, f, i, i, i, vp, vp, vp]
        L.moe_finalize_rmsnorm_mxfp8.restype = i
        L.moe_finalize_rmsnorm_mxfp8.argtypes = [vp, vp, vp, vp, vp, f, i, i, i, vp, vp, vp, vp, vp]
        L.moe_layer_workspace_bytes.restype = sz
        L.moe_layer_workspace_bytes.argtypes = [C.POINTER(moe_layer_desc)]
        L.moe_layer.restype = i
        L.moe_layer.argtypes = [C.POINTER(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_layer_mxfp8_out.restype = i
        L.moe_layer_mxfp8_out.argtypes = [C.POINTER(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          sz, vp]
        L.moe_expert_gate_up_fp8s.restype = i
        L.moe_expert_gate_up_fp8s.argtypes = [C.POINTER(moe_weights), vp, f, f, i, i, i, f, vp, vp, sz, vp]
        L.moe_expert_down_fp8s.restype = i
        L.moe_expert_down_fp8s.argtypes = [C.POINTER(moe_weights), vp, f, i, i, i, vp, vp]
        L.moe_layer_noalloc.restype = i
        L.moe_layer_noalloc.argtypes = [C.POINTER(moe_layer_desc), vp, vp, vp, vp, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the C ABI must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise RuntimeError(f"{what} failed: {lib().moe_status_str(rc).decode()} (status {rc})")


def status_str(rc: int) -> str:
    return lib().moe_status_str(rc).decode()


def abi_version() -> int:
    return lib().moe_abi_version()


def tile_capacity(M: int, E: int, k: int) -> int:
    return lib().moe_tile_capacity(M, E, k)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned device buffer (torch's allocator aligns to 512)."""
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def _call_workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace for one call that the binding drops at return: allocated
    from torch's caching allocator and marked as used by the call's stream, so
    the block is not handed to another allocation before the kernels on that
    stream are done with it."""
    t = workspace(nbytes, device)
    if stream is not None:
        t.record_stream(stream)
    return t


@dataclass
class Weights:
    """One projection of E experts in the canonical layout (see moe.h)."""
    fmt: int
    w: Optional[torch.Tensor] = None
    scales: Optional[torch.Tensor] = None
    global_scale: Optional[torch.Tensor] = None
    packed: bool = False  # FP4: in the load-order layout of moe_pack_fp4

    def c(self) -> moe_weights:
        return moe_weights(self.fmt, _p(self.w), _p(self.scales), _p(self.global_scale))


def _need_packed(*ws: "Weights"):
    for w in ws:
        if w.fmt in (MOE_FMT_MXFP4, MOE_FMT_NVFP4) and not w.packed:
            raise ValueError("FP4 weights must be in the load-order layout: pass them through pack_fp4")


def pack_fp4(w: "Weights", stream=None) -> "Weights":
    """Standard-layout FP4 weights -> the load-order layout the expert GEMMs
    take (moe_pack_fp4); bf16 and absent weights are returned unchanged."""
    if w.fmt not in (MOE_FMT_MXFP4, MOE_FMT_NVFP4):
        return w
    E, N = w.w.shape[0], w.w.shape[1]
    K = 2 * w.w.shape[2]
    nb = lib().moe_packed_scale_bytes(w.fmt, E, N, K)
    if nb == 0:
        raise ValueError(f"unsupported FP4 matrix shape E={E} N={N} K={K}")
    w_out = torch.empty_like(w.w)
    s_out = torch.empty(nb, dtype=torch.uint8, device=w.w.device)
    _check(lib().moe_pack_fp4(w.fmt, E, N, K, _p(w.w), _p(w.scales), _p(w_out), _p(s_out), _stream(stream)),
           "moe_pack_fp4")
    return Weights(w.fmt, w_out, s_out, w.global_scale, packed=True)


class Routing:
    """Device buffers of a routing result (moe_routing)."""

    def __init__(self, M: int, E: int, k: int, device):
        P = M * k
        T = tile_capacity(M, E, k)
        i32 = dict(dtype=torch.int32, device=device)
        self.M, self.E, self.k = M, E, k
        self.topk_ids = torch.empty((M, k), **i32)
        self.topk_w = torch.empty((M, k), dtype=torch.float32, device=device)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.bucket = torch.empty(P, **i32)
        self.tile_expert = torch.empty(T, **i32)
        self.tile_begin = torch.empty(T, **i32)
        self.tile_rows = torch.empty(T, **i32)
        self.num_tiles = torch.empty(1, **i32)
        self.active_experts = torch.empty(min(E, P), **i32)
        self.num_active = torch.empty(1, **i32)
        self.active_offsets = torch.empty(min(E, P) + 1, **i32)

    def c(self) -> moe_routing:
        return moe_routing(*[_p(getattr(self, n)) for n, _ in moe_routing._fields_])


def route_topk(routing: Routing, x=None, logits_in=None, w_router=None, bias=None,
               routed_scale: float = 1.0, logits_out=None, ws=None, stream=None):
    M, E, k = routing.M, routing.E, routing.k
    H = x.shape[1] if x is not None else 0
    dev = (x if x is not None else logits_in).device
    need = lib().moe_route_workspace_bytes(M, H, E, k)
    if ws is None:
        ws = _call_workspace(need, dev, stream)
    r = routing.c()
    rc = lib().moe_route_topk(_p(x), _p(logits_in), _p(w_router), _p(bias), M, H, E, k,
                              float(routed_scale), _p(logits_out), C.byref(r), _p(ws), ws.numel(),
                              _stream(stream))
    _check(rc, "moe_route_topk")


def quant_act_mxfp8(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, routing: Optional["Routing"] = None,
                    stream=None):
    """MXFP8 of the rows of x: row order, or bucket order [M*k, K] with a routing."""
    M, K = x.shape
    r = None if routing is None else routing.c()
    k = 0 if routing is None else routing.k
    _check(lib().moe_quant_act_mxfp8(_p(x), M, K, None if r is None else C.byref(r), k, _p(q), _p(s),
                                     _stream(stream)), "moe_quant_act_mxfp8")


def quant_act_nvfp4(x: torch.Tensor, g: float, q: torch.Tensor, s: torch.Tensor,
                    routing: Optional["Routing"] = None, stream=None):
    """NVFP4 of bf16 rows with global g: q [rows, K/2], s [rows, K/16]."""
    M, K = x.shape
    r = None if routing is None else routing.c()
    rc = lib().moe_quant_act_nvfp4(_p(x), M, K, float(g), None if r is None else C.byref(r),
                                   routing.k if routing is not None else 0, _p(q), _p(s), _stream(stream))
    _check(rc, "moe_quant_act_nvfp4")


def expert_gate_up(w13: Weights, M, H, I, E, k, routing: Optional[Routing] = None, a_q=None,
                   a_s=None, a_bf16=None, h_q=None, h_s=None, h_bf16=None, ws=None, stream=None,
                   swiglu_limit=0.0):
    _need_packed(w13)
    dense = routing is None
    dev = (a_q if a_q is not None else a_bf16).device
    need = lib().moe_gate_up_workspace_bytes(w13.fmt, M, H, I, E, k, int(dense))
    if ws is None and need:
        ws = _call_workspace(need, dev, stream)
    wc = w13.c()
    r = None if dense else routing.c()
    rc = lib().moe_expert_gate_up(C.byref(wc), _p(a_q), _p(a_s), _p(a_bf16),
                                  None if dense else C.byref(r), M, H, I, E, k, float(swiglu_limit),
                                  _p(h_q), _p(h_s),
                                  _p(h_bf16), _p(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "moe_expert_gate_up")


def expert_gate_up_tok(w13: Weights, M, H, I, E, k, routing: Routing, a_q, a_s, h_q, h_s, ws=None, stream=None,
                       swiglu_limit=0.0):
    """Routed gate_up with the MXFP8 activations in token order [M, H]; h in
    bucket order, as expert_gate_up writes it."""
    _need_packed(w13)
    need = lib().moe_gate_up_workspace_bytes(w13.fmt, M, H, I, E, k, 0)
    if ws is None and need:
        ws = _call_workspace(need, a_q.device, stream)
    wc = w13.c()
    r = routing.c()
    rc = lib().moe_expert_gate_up_tok(C.byref(wc), _p(a_q), _p(a_s), C.byref(r), M, H, I, E, k,
                                      float(swiglu_limit), _p(h_q), _p(h_s), _p(ws),
                                      0 if ws is None else ws.numel(), _stream(stream))
    _check(rc, "moe_expert_gate_up_tok")


def expert_down(w2: Weights, M, H, I, E, k, y, routing: Optional[Routing] = None, h_q=None,
                h_s=None, h_bf16=None, stream=None):
    _need_packed(w2)
    wc = w2.c()
    r = None if routing is None else routing.c()
    rc = lib().moe_expert_down(C.byref(wc), _p(h_q), _p(h_s), _p(h_bf16),
                               None if routing is None else C.byref(r), M, H, I, E, k, _p(y),
                               _stream(stream))
    _check(rc, "moe_expert_down")


def expert_gate_up_nvfp4a(w13: Weights, M, H, I, E, k, a_q, a_s, a_global: float, h_globals, h_q, h_s,
                          routing: Optional[Routing] = None, swiglu_limit=0.0, stream=None):
    """gate_up of NVFP4 experts on NVFP4 activations; h written as NVFP4
    with h_globals (device fp32 [E], or [1] without a routing)."""
    _need_packed(w13)
    wc = w13.c()
    r = None if routing is None else routing.c()
    rc = lib().moe_expert_gate_up_nvfp4a(C.byref(wc), _p(a_q), _p(a_s), float(a_global),
                                         None if r is None else C.byref(r), M, H, I, E, k, float(swiglu_limit),
                                         _p(h_globals), _p(h_q), _p(h_s), _stream(stream))
    _check(rc, "moe_expert_gate_up_nvfp4a")


def expert_down_nvfp4a(w2: Weights, M, H, I, E, k, h_q, h_s, h_globals, y, routing: Optional[Routing] = None,
                       stream=None):
    _need_packed(w2)
    wc = w2.c()
    r = None if routing is None else routing.c()
    rc = lib().moe_expert_down_nvfp4a(C.byref(wc), _p(h_q), _p(h_s), _p(h_globals),
                                      None if r is None else C.byref(r), M, H, I, E, k, _p(y), _stream(stream))
    _check(rc, "moe_expert_down_nvfp4a")


def expert_gate_up_fp8s(w13: Weights, M, H, I, x, s_in: float, s_h: float, h_q, swiglu_limit=0.0, ws=None,
                        stream=None):
    """The static-FP8 shared expert's gate_up: h codes [M, I] from bf16 x."""
    need = lib().moe_gate_up_workspace_bytes(MOE_FMT_FP8S, M, H, I, 1, 1, 1)
    if ws is None:
        ws = _call_workspace(need, x.device, stream)
    wc = w13.c()
    rc = lib().moe_expert_gate_up_fp8s(C.byref(wc), _p(x), float(s_in), float(s_h), M, H, I, float(swiglu_limit),
                                       _p(h_q), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "moe_expert_gate_up_fp8s")


def expert_down_fp8s(w2: Weights, M, H, I, h_q, s_h: float, y, stream=None):
    wc = w2.c()
    rc = lib().moe_expert_down_fp8s(C.byref(wc), _p(h_q), float(s_h), M, H, I, _p(y), _stream(stream))
    _check(rc, "moe_expert_down_fp8s")


def finalize_rmsnorm(y, topk_w, y_sh, residual, gamma, eps, out, residual_out=None, stream=None,
                     out_q=None, out_s=None):
    """moe_finalize_rmsnorm; with out_q/out_s, moe_finalize_rmsnorm_mxfp8."""
    M, H = residual.shape
    k = topk_w.shape[1]
    if out_q is None and out_s is None:
        rc = lib().moe_finalize_rmsnorm(_p(y), _p(topk_w), _p(y_sh), _p(residual), _p(gamma),
                                        float(eps), M, H, k, _p(out), _p(residual_out), _stream(stream))
        _check(rc, "moe_finalize_rmsnorm")
        return
    rc = lib().moe_finalize_rmsnorm_mxfp8(_p(y), _p(topk_w), _p(y_sh), _p(residual), _p(gamma),
                                          float(eps), M, H, k, _p(out), _p(residual_out), _p(out_q),
                                          _p(out_s), _stream(stream))
    _check(rc, "moe_finalize_rmsnorm_mxfp8")


class Layer:
    """The fused layer (moe_layer) over weights held in torch device tensors."""

    def __init__(self, M, H, E, k, I, I_sh, routed_scale, eps, w_router, router_bias,
                 w13: Weights, w2: Weights, sh13: Weights, sh2: Weights, gamma, swiglu_limit=0.0,
                 act_fmt=0, x_global=0.0, h_globals=None, sh_h_global=None, sh_in_scale=0.0, sh_h_scale=0.0):
        _need_packed(w13, w2, sh13, sh2)
        self._keep = (w_router, router_bias, w13, w2, sh13, sh2, gamma, h_globals, sh_h_global)
        self.M, self.H, self.E, self.k = M, H, E, k
        self.desc = moe_layer_desc(M, H, E, k, I, I_sh, float(routed_scale), float(eps),
                                   _p(w_router), _p(router_bias), w13.c(), w2.c(), sh13.c(),
                                   sh2.c(), _p(gamma), float(swiglu_limit), int(act_fmt), float(x_global),
                                   _p(h_globals), _p(sh_h_global), float(sh_in_scale), float(sh_h_scale))
        self.ws_bytes = lib().moe_layer_workspace_bytes(C.byref(self.desc))
        if self.ws_bytes == 0:
            raise RuntimeError("moe_layer_workspace_bytes rejected the layer description")
        self.ws = workspace(self.ws_bytes, w_router.device)

    def set_weights(self, w13: Weights, w2: Weights, sh13: Weights, sh2: Weights):
        """Point the layer at another copy of its weights (same shapes)."""
        _need_packed(w13, w2, sh13, sh2)
        self.desc.w13, self.desc.w2, self.desc.sh13, self.desc.sh2 = w13.c(), w2.c(), sh13.c(), sh2.c()
        self._keep = self._keep[:2] + (w13, w2, sh13, sh2) + self._keep[6:]

    def __call__(self, x, residual, out, residual_out=None, logits_out=None, topk_ids_out=None,
                 topk_w_out=None, stream=None, out_q=None, out_s=None):
        """moe_layer; with out_q/out_s, moe_layer_mxfp8_out."""
        if out_q is None and out_s is None:
            rc = lib().moe_layer(C.byref(self.desc), _p(x), _p(residual), _p(out), _p(residual_out),
                                 _p(logits_out), _p(topk_ids_out), _p(topk_w_out), _p(self.ws),
                                 self.ws.numel(), _stream(stream))
            _check(rc, "moe_layer")
            return
        rc = lib().moe_layer_mxfp8_out(C.byref(self.desc), _p(x), _p(residual), _p(out), _p(residual_out),
                                       _p(out_q), _p(out_s), _p(logits_out), _p(topk_ids_out),
                                       _p(topk_w_out), _p(self.ws), self.ws.numel(), _stream(stream))
        _check(rc, "moe_layer_mxfp8_out")


def layer_noalloc(layer: "Layer", x, residual, out, residual_out=None, logits_out=None, topk_ids_out=None,
                  topk_w_out=None, stream=None):
    """moe_layer_noalloc on the description of `layer` (its own workspace is
    not used): the scratch is the library's static per-device buffer."""
    rc = lib().moe_layer_noalloc(C.byref(layer.desc), _p(x), _p(residual), _p(out), _p(residual_out),
                                 _p(logits_out), _p(topk_ids_out), _p(topk_w_out), _stream(stream))
    _check(rc, "moe_layer_noalloc")
