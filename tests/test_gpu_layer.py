"""GPU parity of the fused layer (moe_layer) against the oracle at the five
workload shapes and at edge shapes, plus the layer's invariants: repeated
launches bitwise identical, any row order gives the same bytes per row, and
HIP-graph replay equals eager execution."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_sigmoid_amd import moe, staging, synth
from oracle import oracle as orc
from tests.parity import (DEV, LOGITS_ABS_MAX, MAX_ABS_MAX, REL_L2_MAX, LayerRun, compare_layer, np_of,
                          sample_rows)

pytestmark = pytest.mark.gpu

# rows the oracle recomputes per workload: all of them (wide's 384 rows take
# the threaded oracle about 15 s on 16 host cores); skew samples 10 rows plus
# the rows of its two hottest experts
SAMPLES = {
    "tiny-m4-h1024-e16-k4-mxfp4": 4,
    "verify-m8-h7168-e256-k8-nvfp4": 8,
    "decode-m16-h7168-e384-k8-mxfp4": 16,
    "skew-m48-h4096-e512-k10-nvfp4": 10,
    "wide-m384-h7168-e256-k8-mxfp4": 384,
}

_cache = {}


def _workload(name):
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        inp = synth.make_inputs(name, seed=synth.WORKLOAD_ORDER.index(name) + 1)
        _cache[name] = (inp, staging.to_device(inp, DEV))
    return _cache[name]


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_layer_parity_workload(name):
    inp, d = _workload(name)
    print(f"[layer parity] {name}", flush=True)
    run = LayerRun(d)
    rows = sample_rows(inp.shape.M, SAMPLES[name], seed=1)
    if name.startswith("skew"):
        # include the rows of the hottest experts (multi-tile experts)
        ids = np_of(run.ids)
        hot = np.bincount(ids.ravel(), minlength=inp.shape.E).argsort()[::-1][:2]
        extra = [int(np.nonzero((ids == e).any(axis=1))[0][0]) for e in hot]
        rows = np.array(sorted(set(rows.tolist()) | set(extra)))
    c = compare_layer(inp, run, rows)
    print(f"  rows={len(rows)} rel_l2={c['rel_l2']:.3e} max_abs={c['max_abs']:.3e} "
          f"res_rel_l2={c['res_rel_l2']:.3e} w_rel={c['w_rel']:.2e} logits_err={c['logits_err']:.2e}", flush=True)
    assert c["logits_err"] <= LOGITS_ABS_MAX
    assert c["ids_ok"], (c["ids_gpu"], c["ids_ref"])
    assert c["w_rel"] <= 1e-6
    assert c["rel_l2"] <= REL_L2_MAX and c["max_abs"] <= MAX_ABS_MAX
    assert c["res_rel_l2"] <= REL_L2_MAX


@pytest.mark.parametrize("name", list(synth.EXTRA_WORKLOADS))
def test_layer_parity_extra_workload(name):
    """The further workloads (W4A4 7-row verify) at their full shape, sampled rows."""
    inp = synth.make_inputs(name, seed=synth.seed_of(name))
    d = staging.to_device(inp, DEV)
    print(f"[layer parity] {name}", flush=True)
    run = LayerRun(d)
    c = compare_layer(inp, run, np.arange(inp.shape.M))
    print(f"  rel_l2={c['rel_l2']:.3e} max_abs={c['max_abs']:.3e} res_rel_l2={c['res_rel_l2']:.3e}", flush=True)
    assert c["logits_ok"], c["logits_err"]
    assert c["ids_ok"]
    assert c["rel_l2"] <= REL_L2_MAX and c["max_abs"] <= MAX_ABS_MAX
    assert c["res_rel_l2"] <= REL_L2_MAX


MAX_CASES = [
    dict(M=3, H=16384, E=4, k=2, I=8192, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256),  # largest H and I
    dict(M=4096, H=256, E=4, k=1, I=128, sfmt=synth.MXFP4, I_sh=128),                   # largest M
]


@pytest.mark.parametrize("case", range(len(MAX_CASES)))
def test_layer_parity_max_sizes(case):
    sh = synth.custom_shape(**MAX_CASES[case])
    inp = synth.make_inputs(sh, seed=300 + case, pool_rows=2048)
    print(f"[layer max] {sh.name}", flush=True)
    d = staging.to_device(inp, DEV)
    run = LayerRun(d)
    c = compare_layer(inp, run, sample_rows(sh.M, 8, seed=case))
    print(f"  rel_l2={c['rel_l2']:.3e} max_abs={c['max_abs']:.3e}", flush=True)
    assert c["logits_ok"], c["logits_err"]
    assert c["ids_ok"]
    assert c["rel_l2"] <= REL_L2_MAX and c["max_abs"] <= MAX_ABS_MAX
    assert c["res_rel_l2"] <= REL_L2_MAX


EDGE = [
    dict(M=1, H=128, E=1, k=1, I=128),                                  # smallest layer
    dict(M=5, H=256, E=4, k=4, I=128, bias="normal:0.05"),               # top-k = all experts
    dict(M=37, H=384, E=8, k=2, I=256, sfmt=synth.MXFP4, I_sh=128),     # ragged rows, shared MX
    dict(M=70, H=256, E=3, k=2, I=128, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256),  # >64 rows per expert
    dict(M=9, H=512, E=64, k=6, I=384, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=128, routed_scale=2.5),
    dict(M=130, H=128, E=2, k=1, I=128, bias="zipf:2.0"),               # one expert takes ~all rows
    # the few-pairs path (slots resolved from the ids, two pairs per thread) with one expert
    # taking more than 256 of its 500 pairs
    dict(M=500, H=128, E=2, k=1, I=128, bias="zipf:2.0"),
    # an MXFP4 shared expert of five 32-row passes riding along both routed launches (I > 512),
    # with few pairs (260) and with many (520: the route step's launch)
    dict(M=130, H=256, E=8, k=2, I=640, sfmt=synth.MXFP4, I_sh=640),
    dict(M=130, H=256, E=16, k=4, I=640, sfmt=synth.MXFP4, I_sh=640),
    # the clamped SwiGLU in routed and shared experts (few pairs, many pairs; MX, NV and bf16 shared)
    dict(M=9, H=512, E=64, k=6, I=384, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256, swiglu_limit=0.4),
    dict(M=48, H=1024, E=32, k=8, I=256, wfmt=synth.MXFP4, sfmt=synth.MXFP4, I_sh=256, swiglu_limit=0.5),
    # NVFP4 activations (W4A4): the 7-row verify shape of the pages' Qwen3.5 row with top-10, bf16
    # shared; few pairs with an NVFP4 shared expert; 320 pairs (two per thread) and 576 (bucketed
    # launches), K-streamed down
    dict(M=7, H=1024, E=64, k=10, I=256, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256, act_fmt=synth.ACT_NVFP4),
    dict(M=9, H=512, E=16, k=4, I=384, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=256, act_fmt=synth.ACT_NVFP4),
    dict(M=40, H=768, E=32, k=8, I=640, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=640, act_fmt=synth.ACT_NVFP4,
         swiglu_limit=0.6),
    dict(M=72, H=768, E=32, k=8, I=640, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=640, act_fmt=synth.ACT_NVFP4,
         swiglu_limit=0.6),
    # the static-FP8 shared expert riding the router, top-k and gate_up launches (up to 512 pairs:
    # W4A4 and MXFP8 activations, 320 pairs) or the route step's launch (576 pairs), with the clamp
    dict(M=7, H=1024, E=64, k=10, I=256, wfmt=synth.NVFP4, sfmt=synth.FP8S, I_sh=256, act_fmt=synth.ACT_NVFP4),
    dict(M=9, H=768, E=32, k=4, I=384, wfmt=synth.NVFP4, sfmt=synth.FP8S, I_sh=128),
    dict(M=40, H=512, E=16, k=8, I=256, wfmt=synth.MXFP4, sfmt=synth.FP8S, I_sh=384, swiglu_limit=0.5),
    dict(M=72, H=512, E=16, k=8, I=256, wfmt=synth.MXFP4, sfmt=synth.FP8S, I_sh=384, swiglu_limit=0.5),
    # a bf16 shared expert with 576 pairs (its down rides the route step's launch)
    dict(M=72, H=512, E=32, k=8, I=256, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256),
    # y of 4 MiB or more is written grouped (16-row groups of an expert's rows, column blocks
    # one after another): many pairs, K-streamed down with the MXFP4 shared expert riding (130
    # rows: a 2-row last shared group); few pairs with the down by rows (NVFP4, its shared
    # expert's down a launch of its own), K-streamed MXFP4 with few pairs, and W4A4 both ways
    dict(M=130, H=1024, E=16, k=8, I=640, sfmt=synth.MXFP4, I_sh=640, bias="zipf:1.0"),
    dict(M=60, H=2304, E=32, k=8, I=256, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=256),
    dict(M=50, H=2688, E=16, k=8, I=640, sfmt=synth.MXFP4, I_sh=640),
    dict(M=40, H=3584, E=16, k=8, I=640, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=640, act_fmt=synth.ACT_NVFP4),
    dict(M=60, H=2304, E=32, k=8, I=256, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256, act_fmt=synth.ACT_NVFP4),
    # the 16-row-pass kernels (16 or fewer token rows) with one expert taking nearly every row, in
    # both formats and K-streamed down; 17 rows take the 32-row kernels again
    dict(M=16, H=512, E=8, k=2, I=640, sfmt=synth.MXFP4, I_sh=640, bias="zipf:3.0"),
    dict(M=16, H=512, E=8, k=2, I=640, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=640, bias="zipf:3.0"),
    dict(M=17, H=512, E=8, k=2, I=640, sfmt=synth.MXFP4, I_sh=640, bias="zipf:3.0"),
    # the most experts and the largest top-k the limits allow, on both paths (128 pairs: slots
    # resolved from the ids; 640 pairs: the route step)
    dict(M=4, H=256, E=1024, k=32, I=128),
    dict(M=20, H=256, E=1024, k=32, I=128, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=128),
    # the route step sharing its launch with the shared expert's down (256 threads: chunks of
    # min(128, 1024 / k) rows, the first 4 chunks' ids in registers) past 4 chunks: bf16 shared
    # on MXFP8 and on NVFP4 activations, static-FP8 shared
    dict(M=600, H=256, E=32, k=8, I=128, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=128, bias="zipf:1.0"),
    dict(M=520, H=256, E=16, k=8, I=128, wfmt=synth.MXFP4, sfmt=synth.FP8S, I_sh=128),
    dict(M=600, H=256, E=32, k=8, I=128, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=128, act_fmt=synth.ACT_NVFP4),
    # a small router (router and top-k in one launch, each row's workgroup reading all of W_r)
    # followed by the route step: 600 pairs on MXFP8 activations, 640 on NVFP4 activations
    # at the largest W_r that path takes (E * H = 32768, 64 rows)
    dict(M=60, H=256, E=32, k=10, I=128, sfmt=synth.MXFP4, I_sh=128, bias="zipf:1.0"),
    dict(M=64, H=512, E=64, k=10, I=128, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=128, act_fmt=synth.ACT_NVFP4),
]


@pytest.mark.parametrize("case", range(len(EDGE)))
def test_layer_parity_edge(case):
    sh = synth.custom_shape(**EDGE[case])
    inp = synth.make_inputs(sh, seed=100 + case, pool_rows=4096)
    inp = synth.vary_globals(inp, 7)
    print(f"[layer edge] {sh.name}", flush=True)
    d = staging.to_device(inp, DEV)
    run = LayerRun(d)
    c = compare_layer(inp, run, np.arange(sh.M))
    print(f"  rel_l2={c['rel_l2']:.3e} max_abs={c['max_abs']:.3e}", flush=True)
    assert c["logits_ok"], c["logits_err"]
    assert c["ids_ok"]
    assert c["rel_l2"] <= REL_L2_MAX and c["max_abs"] <= MAX_ABS_MAX
    assert c["res_rel_l2"] <= REL_L2_MAX


def _small_layer(seed=3, a4=False):
    if a4:  # NVFP4 experts on NVFP4 activations, NVFP4 shared expert
        sh = synth.custom_shape(M=24, H=512, E=12, k=3, I=256, wfmt=synth.NVFP4, sfmt=synth.NVFP4,
                                I_sh=128, bias="zipf:1.2", act_fmt=synth.ACT_NVFP4)
    else:
        sh = synth.custom_shape(M=24, H=512, E=12, k=3, I=256, wfmt=synth.MXFP4, sfmt=synth.MXFP4,
                                I_sh=128, bias="zipf:1.2")
    inp = synth.make_inputs(sh, seed=seed, pool_rows=2048)
    return inp, staging.to_device(inp, DEV)


def _router_layer(seed):
    """A router too large for one workgroup per row (partial logits, then the
    top-k launch), with the bf16 shared expert's stages riding those launches."""
    sh = synth.custom_shape(M=24, H=1024, E=128, k=6, I=256, wfmt=synth.NVFP4, sfmt=synth.BF16, I_sh=256,
                            bias="zipf:1.2")
    inp = synth.make_inputs(sh, seed=seed, pool_rows=2048)
    return inp, staging.to_device(inp, DEV)


@pytest.mark.parametrize("case", ["mx", "a4", "router"])
def test_repeated_launches_bitwise_identical(case):
    inp, d = _router_layer(seed=3) if case == "router" else _small_layer(a4=case == "a4")
    first = LayerRun(d)
    ref = first.host()
    for i in range(400):
        first.layer(d.x, d.x, first.out, first.res, first.logits, first.ids, first.w)
    torch.cuda.synchronize()
    h = first.host()
    for k in ref:
        assert np.array_equal(h[k], ref[k]), k
    # and every one of a set of separate launches
    for i in range(20):
        assert np.array_equal(LayerRun(d, layer=first.layer).host()["out"], ref["out"])


def test_row_permutation_invariance():
    """Any order of the same rows gives the same bytes per row (different
    8-row tile maps of the same rows)."""
    inp, d = _small_layer(seed=4)
    base = LayerRun(d).host()
    rng = np.random.default_rng(0)
    for _ in range(3):
        perm = rng.permutation(inp.shape.M)
        xp = d.x.view(torch.int16)[torch.from_numpy(perm).to(DEV)].contiguous()
        run = LayerRun(d, x=xp).host()
        assert np.array_equal(run["out"], base["out"][perm])
        assert np.array_equal(run["res"], base["res"][perm])
        assert np.array_equal(run["ids"], base["ids"][perm])


@pytest.mark.parametrize("case", ["mx", "a4", "router"])
def test_graph_replay_equals_eager(case):
    inp, d = _router_layer(seed=5) if case == "router" else _small_layer(seed=5, a4=case == "a4")
    run = LayerRun(d)
    eager = run.host()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run.layer(d.x, d.x, run.out, run.res, run.logits, run.ids, run.w, stream=s)  # warm up on s
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            run.layer(d.x, d.x, run.out, run.res, run.logits, run.ids, run.w, stream=s)
    for i in range(5):
        run.out.zero_()
        run.res.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        h = run.host()
        for k in eager:
            assert np.array_equal(h[k], eager[k]), (i, k)
        # eager work between replays
        LayerRun(d, layer=run.layer)


@pytest.mark.parametrize("big", [False, True])
def test_layer_mxfp8_next_input(big):
    """moe_layer_mxfp8_out: out, residual_out and routing equal moe_layer's
    bytes, and its MXFP8 output equals the one-pass quant of that out."""
    if big:   # above 256 (row, expert) pairs: the bucketed launch sequence
        sh = synth.custom_shape(M=40, H=1024, E=32, k=8, I=256, wfmt=synth.NVFP4, sfmt=synth.NVFP4, I_sh=128)
    else:
        sh = synth.custom_shape(M=9, H=512, E=64, k=6, I=384, wfmt=synth.MXFP4, sfmt=synth.MXFP4, I_sh=128)
    inp = synth.make_inputs(sh, seed=77 + big, pool_rows=2048)
    d = staging.to_device(inp, DEV)
    print(f"[layer mxfp8 out] {sh.name}", flush=True)
    run = LayerRun(d)
    ref = run.host()
    q = torch.full((sh.M, sh.H), 0x5a, dtype=torch.uint8, device=DEV)
    s = torch.full((sh.M, sh.H // 32), 0x5a, dtype=torch.uint8, device=DEV)
    run.out.zero_()
    run.res.zero_()
    run.layer(d.x, d.x, run.out, run.res, run.logits, run.ids, run.w, out_q=q, out_s=s)
    torch.cuda.synchronize()
    h = run.host()
    for key in ref:
        assert np.array_equal(h[key], ref[key]), key
    rq, rs = orc.mxfp8_quant_bf16(h["out"])
    assert np.array_equal(np_of(s), rs)
    assert np.array_equal(np_of(q), rq)
