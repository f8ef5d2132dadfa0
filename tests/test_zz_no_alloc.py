"""moe_layer_noalloc (the layer on the library's static per-device scratch)
against moe_layer on a workspace of its own: the same bytes in every output,
on two calls in a row, the second with a smaller layer (so it runs over the
first call's leftovers in the shared scratch)."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_sigmoid_amd import moe, staging, synth
from tests.parity import DEV, LayerRun

pytestmark = pytest.mark.gpu


def _noalloc_run(d):
    s = d.shape
    layer = d.layer()
    out = torch.full((s.M, s.H), 0x5a5a, dtype=torch.int16, device=DEV)
    res = torch.full_like(out, 0x5a5a)
    logits = torch.full((s.M, s.E), float("nan"), dtype=torch.float32, device=DEV)
    ids = torch.full((s.M, s.k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((s.M, s.k), float("nan"), dtype=torch.float32, device=DEV)
    moe.layer_noalloc(layer, d.x, d.x, out, res, logits, ids, w)
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy().view(np.uint16), res=res.cpu().numpy().view(np.uint16),
                logits=logits.cpu().numpy(), ids=ids.cpu().numpy(), w=w.cpu().numpy())


def test_noalloc_matches_layer_two_calls_second_smaller():
    # each call needs less scratch than the one before: the skewed-routing
    # workload (48 rows, 480 pairs: the few-pairs launches, a grouped y of
    # 7.5 MiB); 1040 pairs (the route step's launch sequence, a grouped y of
    # 4.1 MiB, the MXFP4 shared expert riding along); the tiny workload (4 rows,
    # 16 pairs, y by pair); then the first again over the smaller calls'
    # leftovers in the shared scratch
    skew = "skew-m48-h4096-e512-k10-nvfp4"
    staged = [(skew, staging.to_device(synth.make_inputs(skew, seed=synth.seed_of(skew)), DEV))]
    mid = synth.custom_shape(M=130, H=1024, E=16, k=8, I=640, sfmt=synth.MXFP4, I_sh=640, bias="zipf:1.0")
    staged.append((mid.name, staging.to_device(synth.make_inputs(mid, seed=41, pool_rows=4096), DEV)))
    tiny = "tiny-m4-h1024-e16-k4-mxfp4"
    staged.append((tiny, staging.to_device(synth.make_inputs(tiny, seed=synth.seed_of(tiny)), DEV)))
    sizes = [d.layer().ws_bytes for _, d in staged]
    assert sizes[0] > sizes[1] > sizes[2], sizes
    for n, d in staged:
        print(f"[noalloc] {n}", flush=True)
        got = _noalloc_run(d)
        ref = LayerRun(d).host()
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (n, key)
    # and the larger one again after the smaller
    n, d = staged[0]
    got = _noalloc_run(d)
    ref = LayerRun(d).host()
    for key in ref:
        assert np.array_equal(got[key], ref[key]), (n, "again", key)


def test_noalloc_refuses_more_than_its_scratch():
    sh = synth.WORKLOADS["wide-m384-h7168-e256-k8-mxfp4"]
    small = synth.custom_shape(M=4, H=256, E=4, k=2, I=128)
    d = staging.to_device(synth.make_inputs(small, seed=1, pool_rows=256), DEV)
    layer = d.layer()
    # the same layer description with the wide step's shape needs 107 MiB
    desc = moe.moe_layer_desc.from_buffer_copy(layer.desc)
    desc.M, desc.H, desc.E, desc.k, desc.I, desc.I_sh = sh.M, sh.H, sh.E, sh.k, sh.I, 0
    import ctypes as C
    rc = moe.lib().moe_layer_noalloc(C.byref(desc), d.x.data_ptr(), d.x.data_ptr(), d.x.data_ptr(), None, None,
                                     None, None, None)
    assert rc == moe.MOE_ERR_SCRATCH
