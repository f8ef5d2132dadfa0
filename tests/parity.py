"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

from block_scaled_fp4_sigmoid_amd import moe, staging, synth
from oracle import oracle as orc

DEV = "cuda"

# Acceptance bars for the layer outputs against the oracle's fp64 values.
REL_L2_MAX = 5e-3
MAX_ABS_MAX = 3e-2
# Router logits (fp32 products of bf16 x and fp32 weights, fp32 sums) against
# the oracle's fp64 logits.
LOGITS_ABS_MAX = 1e-5


def bf16_to_f64(a) -> np.ndarray:
    a = np.asarray(a).astype(np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


class LayerRun:
    """One moe_layer call on device inputs; outputs copied to the host."""

    def __init__(self, dinp: staging.DeviceInputs, layer=None, x=None):
        s = dinp.shape
        self.layer = layer or dinp.layer()
        x = dinp.x if x is None else x
        self.out = torch.empty((s.M, s.H), dtype=torch.int16, device=DEV)
        self.res = torch.empty((s.M, s.H), dtype=torch.int16, device=DEV)
        self.logits = torch.empty((s.M, s.E), dtype=torch.float32, device=DEV)
        self.ids = torch.empty((s.M, s.k), dtype=torch.int32, device=DEV)
        self.w = torch.empty((s.M, s.k), dtype=torch.float32, device=DEV)
        self.layer(x, x, self.out, self.res, self.logits, self.ids, self.w)
        torch.cuda.synchronize()

    def host(self):
        return dict(out=np_of(self.out).view(np.uint16), res=np_of(self.res).view(np.uint16),
                    logits=np_of(self.logits), ids=np_of(self.ids), w=np_of(self.w))


def oracle_rows(inp: synth.MoEInputs, rows, logits: np.ndarray, want_h=False):
    """Oracle outputs of the sampled rows, routed from the given fp32 logits;
    only the experts those rows choose are decoded."""
    sh = inp.shape
    need = set()
    for r in rows:
        ids, _, _ = orc.topk_row(logits[r], inp.bias, sh.k, sh.routed_scale)
        need.update(int(e) for e in ids)
    L = orc.Layer(inp, experts=need)
    return L.rows(np.asarray(rows, np.int32), logits=logits, want_h=want_h)


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1])
    while len(rows) < n:
        rows.add(int(rng.integers(M)))
    return np.array(sorted(rows))


def compare_layer(inp, run: LayerRun, rows):
    """Layer parity on sampled rows: the fused router launch's logits against
    the oracle's fp64 logits, ids bit-exact (oracle routed from the GPU
    logits), out / residual_out within the bars."""
    h = run.host()
    rows = np.asarray(rows)
    ref_logits = orc.router_logits(np.ascontiguousarray(inp.x[rows]), inp.Wr)
    logits_err = float(np.max(np.abs(h["logits"][rows].astype(np.float64) - ref_logits)))
    ref = oracle_rows(inp, rows, h["logits"])
    ids_ok = np.array_equal(h["ids"][rows], ref["ids"])
    w_rel = float(np.max(np.abs(h["w"][rows] - ref["w"]) / np.abs(ref["w"])))
    got = bf16_to_f64(h["out"][rows])
    r_l2 = rel_l2(got, ref["out64"])
    mabs = float(np.max(np.abs(got - ref["out64"])))
    res_got = bf16_to_f64(h["res"][rows])
    res_ref = bf16_to_f64(ref["resid_out"])
    res_l2 = rel_l2(res_got, res_ref)
    return dict(ids_ok=ids_ok, w_rel=w_rel, rel_l2=r_l2, max_abs=mabs, res_rel_l2=res_l2,
                ids_gpu=h["ids"][rows], ids_ref=ref["ids"], logits_err=logits_err,
                logits_ok=logits_err <= LOGITS_ABS_MAX)
