"""GPU parity of each step of the layer against the oracle, through the C ABI,
on identical seeded inputs: quant bytes and routing bit-exact, expert GEMMs
and finalize within bars derived from their arithmetic."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_sigmoid_amd import moe, staging, synth
from oracle import oracle as orc
from tests.parity import DEV, bf16_to_f64, np_of, rel_l2

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(synth._bf16_trunc(np.asarray(a, np.float32)).view(np.int16)).to(DEV)


def test_quant_mxfp8_bitexact():
    rng = np.random.default_rng(0)
    M, K = 37, 1024  # ragged row count
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (M, K // 32, 1))).repeat(32, 2).reshape(M, K)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[1, :32] = 1e-39               # bf16 subnormals
    x[2, 5] = np.nan
    x[3, 70] = np.inf
    x[4, :32] = 448 * 2.0 ** 10     # exactly at the saturation edge after scaling
    xb = synth._bf16_trunc(x)
    xt = torch.from_numpy(xb.view(np.int16)).to(DEV)
    q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    moe.quant_act_mxfp8(xt, q, s)
    torch.cuda.synchronize()
    rq, rs = orc.mxfp8_quant_bf16(xb)
    assert np.array_equal(np_of(s), rs)
    assert np.array_equal(np_of(q), rq)


@pytest.mark.parametrize("routed", [False, True])
def test_quant_nvfp4_bitexact(routed):
    """NVFP4 activations, byte for byte against the oracle's rule (both sides
    decide every code in fp32), in row order and in bucket order."""
    rng = np.random.default_rng(11)
    M, K = 37, 1024  # ragged row count
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (M, K // 16, 1))).repeat(16, 2).reshape(M, K)
    x[0, :16] = 0.0
    x[0, 16:32] = -0.0
    x[1, :16] = 1e-39               # bf16 subnormals
    x[2, 5] = np.nan
    x[3, 70] = np.inf
    x[4, :16] = 1e30                # scale saturates at 448, codes at 6
    x[5, 32:48] = np.float32(6 * 448) * np.float32(0.01)
    xb = synth._bf16_trunc(x)
    xt = torch.from_numpy(xb.view(np.int16)).to(DEV)
    g = float(np.float32(0.0123))
    if routed:
        E, k = 8, 3
        rt = moe.Routing(M, E, k, DEV)
        logits = torch.from_numpy(rng.standard_normal((M, E)).astype(np.float32)).to(DEV)
        moe.route_topk(rt, logits_in=logits)
        rows = M * k
    else:
        rt, rows = None, M
    q = torch.full((rows, K // 2), 0x5a, dtype=torch.uint8, device=DEV)
    s = torch.full((rows, K // 16), 0x5a, dtype=torch.uint8, device=DEV)
    moe.quant_act_nvfp4(xt, g, q, s, routing=rt)
    torch.cuda.synchronize()
    rq, rs = orc.nvfp4_quant_bf16(xb, g)
    if routed:
        tok = np_of(rt.bucket) // k
        rq, rs = rq[tok], rs[tok]
    assert np.array_equal(np_of(s), rs)
    assert np.array_equal(np_of(q), rq)


ROUTE_CASES = [
    # M, H, E, k, bias, scale
    (4, 1024, 16, 4, "normal:0.01", 1.0),
    (8, 7168, 256, 8, "none", 2.5),
    (48, 4096, 512, 10, "zipf:1.2", 1.0),
    (384, 7168, 256, 8, "none", 1.0),
    (1, 128, 1, 1, "none", 1.0),       # E = k = 1
    (5, 256, 7, 7, "normal:0.05", 1.0),  # k = E
    (100, 384, 3, 2, "none", 1.0),     # few experts, many rows per expert
    (37, 640, 1024, 32, "none", 1.0),  # largest E and k
    (16, 7168, 384, 8, "none", 1.0),   # the decode workload's router
    # the router's K chunks in pairs of software-pipelined rounds: two pairs of
    # 128-K rounds (M <= 16) and three pairs of 64-K rounds (M <= 16, chunks of 384)
    (8, 8192, 1024, 8, "none", 1.0),
    (12, 6144, 1024, 8, "normal:0.01", 1.0),
    # the route step of its own launch (1024 threads) places rows in chunks of
    # min(384, 4096 / k) rows (four pairs per thread) and keeps the first 4
    # chunks' expert ids in registers; the last three run past 4 chunks
    (1024, 512, 64, 8, "zipf:1.0", 1.0),  # 3 chunks of 384 rows (the last ragged)
    (600, 512, 64, 10, "zipf:1.0", 1.0),  # 2 chunks of 384 rows
    (4096, 256, 4, 1, "none", 1.0),       # 11 chunks of 384 rows
    (2000, 256, 64, 8, "zipf:1.0", 1.0),  # 6 chunks of 384 rows (the last 80)
    (700, 128, 64, 32, "none", 1.0),      # 6 chunks of 128 rows (the last 60)
]


@pytest.mark.parametrize("M,H,E,k,bias,scale", ROUTE_CASES)
def test_route_topk_parity(M, H, E, k, bias, scale):
    sh = synth.custom_shape(M=M, H=H, E=E, k=k, I=128, bias=bias, routed_scale=scale)
    inp = synth.make_inputs(sh, seed=M + E, pool_rows=16)
    x = torch.from_numpy(inp.x.view(np.int16)).to(DEV)
    Wr = torch.from_numpy(inp.Wr).to(DEV)
    bias_t = None if inp.bias is None else torch.from_numpy(inp.bias).to(DEV)
    rt = moe.Routing(M, E, k, DEV)
    logits = torch.empty((M, E), dtype=torch.float32, device=DEV)
    moe.route_topk(rt, x=x, w_router=Wr, bias=bias_t, routed_scale=scale, logits_out=logits)
    torch.cuda.synchronize()
    lg = np_of(logits)
    ref64 = orc.router_logits(inp.x, inp.Wr)
    assert np.max(np.abs(lg - ref64)) <= 1e-5
    r = orc.route(lg, inp.bias, k, scale)  # oracle routing on identical fp32 logits
    assert np.array_equal(np_of(rt.topk_ids), r["ids"])
    assert np.max(np.abs(np_of(rt.topk_w) - r["w"]) / np.abs(r["w"])) <= 1e-6
    assert np.array_equal(np_of(rt.expert_offsets), r["offsets"])
    assert np.array_equal(np_of(rt.bucket), r["bucket"])
    nt = int(np_of(rt.num_tiles)[0])
    assert nt == r["num_tiles"]
    assert np.array_equal(np_of(rt.tile_expert)[:nt], r["tile_expert"])
    assert np.array_equal(np_of(rt.tile_begin)[:nt], r["tile_begin"])
    assert np.array_equal(np_of(rt.tile_rows)[:nt], r["tile_rows"])
    counts = np.diff(r["offsets"])
    act = np.nonzero(counts)[0]
    na = int(np_of(rt.num_active)[0])
    assert na == len(act) and np.array_equal(np_of(rt.active_experts)[:na], act)
    # slot ranges: the active experts' offsets, then P for every unused slot
    U = min(E, M * k)
    want = np.full(U + 1, M * k, dtype=np.int64)
    want[:na] = r["offsets"][act]
    assert np.array_equal(np_of(rt.active_offsets), want)
    # routing from logits_in gives the same result
    rt2 = moe.Routing(M, E, k, DEV)
    moe.route_topk(rt2, logits_in=logits, bias=bias_t, routed_scale=scale)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_w", "expert_offsets", "bucket"):
        assert torch.equal(getattr(rt, name), getattr(rt2, name)), name


TIE_CASES = [
    # E, k: list lengths per lane of 1..16 keys and their edges
    (16, 4), (64, 8), (65, 8), (200, 8), (256, 8), (257, 10), (384, 8), (512, 32), (513, 8),
    (1000, 32), (1024, 32), (1024, 1),
]


@pytest.mark.parametrize("E,k", TIE_CASES)
def test_route_topk_ties(E, k):
    """Top-k on logits with many exactly equal scores, negative keys (a
    bias below -1) and keys that tie across the bias: equal keys go to the
    smaller expert id, as in the oracle."""
    M = 5
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(M, E)).astype(np.float32)
    bias = rng.choice(np.array([-2.0, 0.0, 0.25], np.float32), size=E).astype(np.float32)
    for b in (None, bias):
        rt = moe.Routing(M, E, k, DEV)
        moe.route_topk(rt, logits_in=torch.from_numpy(lg).to(DEV),
                       bias=None if b is None else torch.from_numpy(b).to(DEV), routed_scale=1.0)
        torch.cuda.synchronize()
        r = orc.route(lg, b, k, 1.0)
        assert np.array_equal(np_of(rt.topk_ids), r["ids"])
        assert np.max(np.abs(np_of(rt.topk_w) - r["w"]) / np.abs(r["w"])) <= 1e-6
        assert np.array_equal(np_of(rt.bucket), r["bucket"])


def _negate_some_scales(inp, seed):
    """Set the sign bit of about a quarter of the NVFP4 block-scale codes: a
    negative E4M3 scale is a legal code and negates its block."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for pe in (inp.w13, inp.w2):
        flip = rng.random(pe.pool_scales.shape) < 0.25
        pe.pool_scales = np.where(flip, pe.pool_scales | np.uint8(0x80), pe.pool_scales).astype(np.uint8)
    return inp


def _routed_setup(wfmt, M=40, H=512, E=6, k=3, I=256, seed=3, bias="zipf:1.0", neg_scales=False):
    sh = synth.custom_shape(M=M, H=H, E=E, k=k, I=I, wfmt=wfmt, bias=bias)
    inp = synth.make_inputs(sh, seed=seed, pool_rows=2048)
    inp = synth.vary_globals(inp, seed + 1)
    if neg_scales:
        inp = _negate_some_scales(inp, seed + 2)
    d = staging.to_device(inp, DEV)
    rt = moe.Routing(M, E, k, DEV)
    logits = torch.empty((M, E), dtype=torch.float32, device=DEV)
    moe.route_topk(rt, x=d.x, w_router=d.Wr, bias=d.bias, routed_scale=sh.routed_scale, logits_out=logits)
    # row order (what the oracle reads) and bucket order (what the routed GEMMs read)
    xq = torch.empty((M, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty((M, H // 32), dtype=torch.uint8, device=DEV)
    moe.quant_act_mxfp8(d.x, xq, xs)
    xqp = torch.empty((M * k, H), dtype=torch.uint8, device=DEV)
    xsp = torch.empty((M * k, H // 32), dtype=torch.uint8, device=DEV)
    moe.quant_act_mxfp8(d.x, xqp, xsp, routing=rt)
    torch.cuda.synchronize()
    # bucket order is row order permuted: row b = row bucket[b] // k, bit for bit
    tok = torch.div(rt.bucket.long(), k, rounding_mode="floor")
    assert torch.equal(xqp, xq[tok]) and torch.equal(xsp, xs[tok])
    return sh, inp, d, rt, (xq, xs), (xqp, xsp)


@pytest.mark.parametrize("wfmt,H,neg,limit", [(synth.MXFP4, 512, False, 0.0), (synth.NVFP4, 512, False, 0.0),
                                              (synth.MXFP4, 2560, False, 0.0), (synth.NVFP4, 2560, False, 0.0),
                                              (synth.NVFP4, 2560, True, 0.0), (synth.MXFP4, 512, False, 0.5),
                                              (synth.NVFP4, 2560, False, 0.5), (synth.MXFP4, 2560, False, 0.5)])
def test_gate_up_routed_parity(wfmt, H, neg, limit):
    # H = 512 is one K chunk; 2560 is five (exercises the weight ring and LDS buffers);
    # limit > 0: the clamped SwiGLU (gate values here have a std of 0.45 to 1)
    sh, inp, d, rt, (xq, xs), (xqp, xsp) = _routed_setup(wfmt, H=H, neg_scales=neg)
    M, H, E, k, I = sh.M, sh.H, sh.E, sh.k, sh.I
    P = M * k
    hq = torch.empty((P, I), dtype=torch.uint8, device=DEV)
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device=DEV)
    moe.expert_gate_up(d.w13, M, H, I, E, k, routing=rt, a_q=xqp, a_s=xsp, h_q=hq, h_s=hs, swiglu_limit=limit)
    # the same rows read in token order through the bucket: the same h bytes
    hq2 = torch.full_like(hq, 0x5a)
    hs2 = torch.full_like(hs, 0x5a)
    moe.expert_gate_up_tok(d.w13, M, H, I, E, k, rt, xq, xs, hq2, hs2, swiglu_limit=limit)
    torch.cuda.synchronize()
    assert torch.equal(hq2, hq) and torch.equal(hs2, hs)
    bucket, ids = np_of(rt.bucket), np_of(rt.topk_ids).ravel()
    a = orc.mxfp8_dequant(np_of(xq), np_of(xs))
    ghq, ghs = np_of(hq), np_of(hs)
    eq_bytes, tot = 0, 0
    worst = 0.0
    for b in range(P):
        p = bucket[b]
        e, r = ids[p], p // k
        m13 = inp.w13.expert(e)
        h = orc.gate_up(orc.Mat(m13.fmt, m13.packed, m13.scales, m13.gscale), H, I, a[r], limit)
        rq, rs = orc.mxfp8_quant_f64(h[None, :])
        eq_bytes += int(np.sum(rq[0] == ghq[b])) + int(np.sum(rs[0] == ghs[b]))
        tot += I + I // 32
        # a flipped code is one E4M3 step at a rounding midpoint of fp32 vs fp64 h
        hd = orc.mxfp8_dequant(ghq[b:b + 1], ghs[b:b + 1])[0]
        worst = max(worst, rel_l2(hd, orc.mxfp8_dequant(rq, rs)[0]))
    assert eq_bytes / tot >= 0.999, eq_bytes / tot
    assert worst < 1e-2, worst


@pytest.mark.parametrize("wfmt,I,neg,H", [(synth.MXFP4, 256, False, 512), (synth.NVFP4, 256, False, 512),
                                          (synth.MXFP4, 1536, False, 512), (synth.NVFP4, 1536, False, 512),
                                          (synth.NVFP4, 256, True, 512), (synth.NVFP4, 1536, True, 512),
                                          (synth.MXFP4, 128, False, 512), (synth.NVFP4, 384, False, 512),
                                          (synth.MXFP4, 512, False, 512), (synth.NVFP4, 512, True, 512),
                                          (synth.MXFP4, 1536, False, 640)])
def test_down_routed_parity(wfmt, I, neg, H):
    # I <= 512 (one quad of K steps) streams along the output rows; 1536 along
    # K (MXFP4: four 16-row blocks per wave when H is a multiple of 256, else
    # two, as at H = 640)
    sh, inp, d, rt, (xq, xs), (xqp, xsp) = _routed_setup(wfmt, H=H, seed=5, I=I, neg_scales=neg)
    M, H, E, k, I = sh.M, sh.H, sh.E, sh.k, sh.I
    P = M * k
    hq = torch.empty((P, I), dtype=torch.uint8, device=DEV)
    hs = torch.empty((P, I // 32), dtype=torch.uint8, device=DEV)
    moe.expert_gate_up(d.w13, M, H, I, E, k, routing=rt, a_q=xqp, a_s=xsp, h_q=hq, h_s=hs)
    y = torch.full((P, H), float("nan"), dtype=torch.float32, device=DEV)
    moe.expert_down(d.w2, M, H, I, E, k, y, routing=rt, h_q=hq, h_s=hs)
    torch.cuda.synchronize()
    bucket, ids = np_of(rt.bucket), np_of(rt.topk_ids).ravel()
    hd = orc.mxfp8_dequant(np_of(hq), np_of(hs))
    gy = np_of(y)
    worst = 0.0
    for b in range(P):
        p = bucket[b]
        m2 = inp.w2.expert(ids[p])
        yr = orc.down(orc.Mat(m2.fmt, m2.packed, m2.scales, m2.gscale), H, I, hd[b])
        worst = max(worst, rel_l2(gy[p], yr))
    assert worst < 2e-3, worst


@pytest.mark.parametrize("I", [256, 1536])
def test_down_nvfp4_outlier_blocks(I):
    """NVFP4 weights on MXFP8 activations whose blocks lie far below the row's
    largest one.  The f16 operand of a value is its E4M3 code times
    2^(its scale - the row's largest scale over the item's K range), which is
    exact unless it falls below f16's smallest normal 2^-14 (then it is
    rounded or flushed: an error of at most the value itself).  So each output
    is within sum_n |W[c, n]| |a_n| [a_n < 2^-14 of the row's largest block
    scale] of the exact fp64 sum, plus the summation's rounding; rows without
    an outlier keep the ordinary accuracy.  I = 256 streams along the output rows, 1536
    along K."""
    sh, inp, d, rt, _, _ = _routed_setup(synth.NVFP4, H=512, seed=9, I=I)
    M, H, E, k, I = sh.M, sh.H, sh.E, sh.k, sh.I
    P, nb = M * k, I // 32
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 256, (P, I)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3F            # no NaN codes
    scales = (118 + rng.integers(0, 4, (P, nb))).astype(np.uint8)
    jump = np.array([0, 12, 20, 40])[np.arange(P) % 4]   # binades of the one outlier block per row
    scales[np.arange(P), rng.integers(0, nb, P)] += jump.astype(np.uint8)
    hq = torch.from_numpy(codes).to(DEV)
    hs = torch.from_numpy(scales).to(DEV)
    y = torch.full((P, H), float("nan"), dtype=torch.float32, device=DEV)
    moe.expert_down(d.w2, M, H, I, E, k, y, routing=rt, h_q=hq, h_s=hs)
    torch.cuda.synchronize()
    bucket, ids = np_of(rt.bucket), np_of(rt.topk_ids).ravel()
    a = orc.mxfp8_dequant(codes, scales)
    gy = np_of(y).astype(np.float64)
    lossy_rows = 0
    for b in range(P):
        p = bucket[b]
        m2 = inp.w2.expert(ids[p])
        mat = orc.Mat(m2.fmt, m2.packed, m2.scales, m2.gscale)
        W = orc.mat_dequant(mat, H, I)
        yr = W @ a[b]
        unit = 2.0 ** (int(scales[b].max()) - 127)
        lost = np.where(np.abs(a[b]) < 2.0 ** -14 * unit, np.abs(a[b]), 0.0)
        lossy_rows += int(np.any(lost > 0))
        # the matrix instruction's sums: 2^-12 of the sum of |products| (the
        # reduced internal precision bound used for the FP8 instruction)
        bound = np.abs(W) @ lost + 2.0 ** -12 * (np.abs(W) @ np.abs(a[b]))
        err = np.abs(gy[p] - yr)
        assert np.all(err <= bound), (b, jump[b], float(np.max(err / bound)))
        assert np.all(np.isfinite(gy[p]))
        if jump[b] == 0:
            assert rel_l2(gy[p], yr) < 5e-4
    assert lossy_rows >= P // 4  # the 20- and 40-binade rows reach below f16's normal range


@pytest.mark.parametrize("sfmt,M,limit", [(synth.MXFP4, 23, 0.0), (synth.NVFP4, 23, 0.0), (synth.MXFP4, 70, 0.0),
                                          (synth.NVFP4, 70, 0.0), (synth.MXFP4, 23, 0.3), (synth.NVFP4, 70, 0.3)])
def test_dense_fp4_expert_parity(sfmt, M, limit):
    """The shared-expert path: one FP4 expert over all rows in order (70 rows:
    three passes of 32 rows, each its own workgroups)."""
    H, I = 384, 256
    sh = synth.custom_shape(M=M, H=H, E=1, k=1, I=128, wfmt=synth.MXFP4, sfmt=sfmt, I_sh=I)
    inp = synth.make_inputs(sh, seed=8, pool_rows=64)
    d = staging.to_device(inp, DEV)
    xq = torch.empty((M, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty((M, H // 32), dtype=torch.uint8, device=DEV)
    moe.quant_act_mxfp8(d.x, xq, xs)
    hq = torch.empty((M, I), dtype=torch.uint8, device=DEV)
    hs = torch.empty((M, I // 32), dtype=torch.uint8, device=DEV)
    moe.expert_gate_up(d.sh13, M, H, I, 1, 1, routing=None, a_q=xq, a_s=xs, h_q=hq, h_s=hs, swiglu_limit=limit)
    y = torch.empty((M, H), dtype=torch.float32, device=DEV)
    moe.expert_down(d.sh2, M, H, I, 1, 1, y, routing=None, h_q=hq, h_s=hs)
    torch.cuda.synchronize()
    a = orc.mxfp8_dequant(np_of(xq), np_of(xs))
    m13 = orc.Mat.from_synth(inp.sh13)
    m2 = orc.Mat.from_synth(inp.sh2)
    ghq, ghs, gy = np_of(hq), np_of(hs), np_of(y)
    hd = orc.mxfp8_dequant(ghq, ghs)
    eq = 0
    for r in range(M):
        h = orc.gate_up(m13, H, I, a[r], limit)
        rq, rs = orc.mxfp8_quant_f64(h[None, :])
        eq += int(np.sum(rq[0] == ghq[r]))
        yr = orc.down(m2, H, I, hd[r])
        assert rel_l2(gy[r], yr) < 2e-3
    assert eq / (M * I) >= 0.999


@pytest.mark.parametrize("M,H,I,limit", [(48, 1024, 256, 0.0), (8, 7168, 256, 0.0), (48, 4096, 512, 0.0),
                                         (8, 7168, 256, 0.8)])
def test_dense_bf16_expert_parity(M, H, I, limit):
    sh = synth.custom_shape(M=M, H=H, E=1, k=1, I=128, sfmt=synth.BF16, I_sh=I)
    inp = synth.make_inputs(sh, seed=9, pool_rows=64)
    d = staging.to_device(inp, DEV)
    hb = torch.empty((M, I), dtype=torch.int16, device=DEV)
    moe.expert_gate_up(d.sh13, M, H, I, 1, 1, routing=None, a_bf16=d.x, h_bf16=hb, swiglu_limit=limit)
    y = torch.empty((M, H), dtype=torch.float32, device=DEV)
    moe.expert_down(d.sh2, M, H, I, 1, 1, y, routing=None, h_bf16=hb)
    torch.cuda.synchronize()
    m13 = orc.Mat.from_synth(inp.sh13)
    m2 = orc.Mat.from_synth(inp.sh2)
    ghb = np_of(hb).view(np.uint16)
    gy = np_of(y)
    eq = 0
    for r in range(M):
        h = orc.gate_up_bf16(m13, H, I, inp.x[r], limit)
        hb_ref = orc.bf16_rne_n(h)
        eq += int(np.sum(hb_ref == ghb[r]))
        yr = orc.down(m2, H, I, bf16_to_f64(ghb[r]))
        assert rel_l2(gy[r], yr) < 1e-5
    assert eq / (M * I) >= 0.99


@pytest.mark.parametrize("M,H,I,limit", [(7, 4096, 512, 0.0), (48, 1024, 256, 0.0), (16, 7168, 2048, 0.0),
                                         (70, 512, 256, 0.5)])
def test_dense_fp8s_expert_parity(M, H, I, limit):
    """The static-FP8 shared expert: h codes (SiLU-and-mul fused with the
    static FP8 quant of the down input) against the oracle's codes, and y
    against the oracle's down on the GPU's own codes (exact products, fp32
    sums).  Codes can differ where the fp32 sums and the fp64 ones round g, u
    or h to bf16 on either side of a midpoint."""
    sh = synth.custom_shape(M=M, H=H, E=1, k=1, I=128, sfmt=synth.FP8S, I_sh=I)
    inp = synth.make_inputs(sh, seed=19, pool_rows=64)
    d = staging.to_device(inp, DEV)
    hq = torch.full((M, I), 0x5a, dtype=torch.uint8, device=DEV)
    moe.expert_gate_up_fp8s(d.sh13, M, H, I, d.x, inp.sh_in13, inp.sh_in2, hq, swiglu_limit=limit)
    y = torch.empty((M, H), dtype=torch.float32, device=DEV)
    moe.expert_down_fp8s(d.sh2, M, H, I, hq, inp.sh_in2, y)
    torch.cuda.synchronize()
    m13, m2 = orc.Mat.from_synth(inp.sh13), orc.Mat.from_synth(inp.sh2)
    e4 = orc.e4m3_table()
    W2abs = np.abs(orc.mat_dequant(m2, H, I))
    sh_ = np.float64(np.float32(inp.sh_in2))
    ghq, gy = np_of(hq), np_of(y)
    eq, worst, l2 = 0, 0.0, 0.0
    for r in range(M):
        h, _ = orc.gate_up_fp8s(m13, H, I, inp.x[r], inp.sh_in13, limit)
        _, hq_ref = orc.down_fp8s(m2, H, I, h, inp.sh_in2)
        eq += int(np.sum(hq_ref == ghq[r]))
        hv = e4[ghq[r]]
        yr = orc.down(m2, H, I, hv) * sh_
        # the fp8 matrix instruction adds its 32 products with a reduced
        # internal precision: bound each output by 2^-12 of its sum of |products|
        bound = 2.0 ** -12 * (W2abs @ np.abs(hv)) * sh_ + 1e-30
        worst = max(worst, float(np.max(np.abs(gy[r] - yr) / bound)))
        l2 = max(l2, rel_l2(gy[r], yr))
    print(f"  h codes equal: {eq / (M * I):.5f}; y: rel_l2 {l2:.2e}, worst error / bound {worst:.3f}")
    assert worst <= 1.0 and l2 < 2e-4
    assert eq / (M * I) >= 0.99


@pytest.mark.parametrize("M,H,k", [
    (19, 2048 + 128, 5),
    # many rows; two column passes per thread at 8576 (the second ragged)
    # and 16384 columns
    (300, 8192 + 384, 3),
    (260, 16384, 2),
])
def test_finalize_parity(M, H, k):
    rng = np.random.default_rng(4 + M)
    y = rng.standard_normal((M * k, H)).astype(np.float32)
    w = rng.random((M, k)).astype(np.float32)
    ysh = rng.standard_normal((M, H)).astype(np.float32)
    res = synth._bf16_trunc(rng.standard_normal((M, H)).astype(np.float32))
    gamma = synth._bf16_trunc((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    t = lambda a: torch.from_numpy(a).to(DEV)
    out = torch.empty((M, H), dtype=torch.int16, device=DEV)
    ro = torch.empty((M, H), dtype=torch.int16, device=DEV)
    moe.finalize_rmsnorm(t(y), t(w), t(ysh), t(res.view(np.int16)), t(gamma.view(np.int16)), 1e-6, out, ro)
    torch.cuda.synchronize()
    go, gr = np_of(out).view(np.uint16), np_of(ro).view(np.uint16)
    for r in range(M):
        o64, ob, rb = orc.finalize_row(y[r * k:(r + 1) * k].astype(np.float64), w[r],
                                       ysh[r].astype(np.float64), res[r], gamma, 1e-6)
        # the fp32 sum differs from the fp64 one by ~1e-7 of the summed magnitudes,
        # so residual_out may take the neighbouring bf16 value at a rounding
        # midpoint, or differ more where the sum cancels to near zero
        mag = np.abs(bf16_to_f64(res[r])) + np.abs(ysh[r]) + np.abs(w[r]) @ np.abs(y[r * k:(r + 1) * k])
        diff = np.abs(bf16_to_f64(gr[r]) - bf16_to_f64(rb))
        allowed = np.abs(bf16_to_f64(rb)) * 2.0 ** -7 + 1e-6 * mag
        assert np.all(diff <= allowed) and (gr[r] != rb).mean() < 0.01
        assert rel_l2(bf16_to_f64(go[r]), o64) < 4e-3
        assert np.max(np.abs(bf16_to_f64(go[r]) - o64)) < 3e-2


@pytest.mark.parametrize("fmt,N,K", [(synth.MXFP4, 48, 640), (synth.NVFP4, 32, 384),
                                     (synth.MXFP4, 16, 1024), (synth.NVFP4, 64, 2048)])
def test_pack_fp4_layout(fmt, N, K):
    """moe_pack_fp4 against the layout written out in moe.h (numpy, byte by byte);
    K = 640 and 384 leave a partial last quad (zero entries)."""
    E = 3
    S, Q = K // 128, (K // 128 + 3) // 4
    rng = np.random.default_rng(N + K)
    nb = K // (32 if fmt == synth.MXFP4 else 16)
    w = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 256, (E, N, nb), dtype=np.uint8)
    g = torch.ones(E, dtype=torch.float32, device=DEV)
    P = moe.pack_fp4(moe.Weights(fmt, torch.from_numpy(w).to(DEV), torch.from_numpy(sc).to(DEV), g))
    torch.cuda.synchronize()
    pw = np_of(P.w).reshape(E, N // 16, S, 64, 16)
    ps = np_of(P.scales)
    for e in range(E):
        for rb in range(N // 16):
            for l in range(64):
                i, gg = l % 16, l // 16
                row = 16 * rb + i
                for st in range(S):
                    assert np.array_equal(pw[e, rb, st, l], w[e, row, 64 * st + 16 * gg:64 * st + 16 * gg + 16])
    if fmt == synth.MXFP4:
        ps = ps.reshape(E, N // 16, Q, 64, 4)
        for e, rb, q, l, u in np.ndindex(E, N // 16, Q, 64, 4):
            i, gg = l % 16, l // 16
            want = sc[e, 16 * rb + i, 4 * (4 * q + u) + gg] if 4 * q + u < S else 0
            assert ps[e, rb, q, l, u] == want
    else:
        ps = ps.reshape(E, N // 16, Q, 64, 8)
        for e, rb, q, l, u, h in np.ndindex(E, N // 16, Q, 64, 4, 2):
            i, gg = l % 16, l // 16
            want = sc[e, 16 * rb + i, 8 * (4 * q + u) + 2 * gg + h] if 4 * q + u < S else 0
            assert ps[e, rb, q, l, 2 * u + h] == want


@pytest.mark.parametrize("M,H", [(19, 2048 + 128), (3, 8192 + 384), (257, 8192 + 384)])
def test_finalize_mxfp8_next_input(M, H):
    """The finalize's MXFP8 of its own bf16 output equals the one-pass quant of
    that output byte for byte; out and residual_out equal the plain call's."""
    rng = np.random.default_rng(40 + M)
    k = 5
    y = rng.standard_normal((M * k, H)).astype(np.float32)
    w = rng.random((M, k)).astype(np.float32)
    ysh = rng.standard_normal((M, H)).astype(np.float32)
    r32 = rng.standard_normal((M, H)).astype(np.float32)
    r32[1, 40] = np.inf      # the whole normed row turns 0 / NaN: the NaN block's scale is 0xFF
    res = synth._bf16_trunc(r32)
    g32 = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    g32[:32] = 0.0           # an all-zero block
    g32[64:96] *= 2.0 ** 20
    gamma = synth._bf16_trunc(g32)
    t = lambda a: torch.from_numpy(a).to(DEV)
    out = torch.empty((M, H), dtype=torch.int16, device=DEV)
    ro = torch.empty((M, H), dtype=torch.int16, device=DEV)
    out2, ro2 = torch.empty_like(out), torch.empty_like(ro)
    q = torch.full((M, H), 0x5a, dtype=torch.uint8, device=DEV)
    s = torch.full((M, H // 32), 0x5a, dtype=torch.uint8, device=DEV)
    args = (t(y), t(w), t(ysh), t(res.view(np.int16)), t(gamma.view(np.int16)), 1e-6)
    moe.finalize_rmsnorm(*args, out, ro)
    moe.finalize_rmsnorm(*args, out2, ro2, out_q=q, out_s=s)
    torch.cuda.synchronize()
    go = np_of(out2).view(np.uint16)
    assert np.array_equal(go, np_of(out).view(np.uint16))
    assert np.array_equal(np_of(ro2), np_of(ro))
    rq, rs = orc.mxfp8_quant_bf16(go)
    assert np.array_equal(np_of(s), rs)
    assert np.array_equal(np_of(q), rq)
    assert (rs[1] == 0xFF).any()
    # E4M3 keeps three mantissa bits: every normal element lies within 2^-4 of
    # its value relative, so the dequantized row is that close to the oracle's
    deq = orc.mxfp8_dequant(np_of(q), np_of(s))
    for r in (0, M - 1):
        o64 = orc.finalize_row(y[r * k:(r + 1) * k].astype(np.float64), w[r], ysh[r].astype(np.float64),
                               res[r], gamma, 1e-6)[0]
        assert rel_l2(deq[r], o64) < 2.0 ** -4


# ---- NVFP4 activations (W4A4) ---------------------------------------------------

def _a4_setup(M, H, E, k, I, seed, I_sh=0, sfmt=synth.NONE, limit=0.0):
    sh = synth.custom_shape(M=M, H=H, E=E, k=k, I=I, wfmt=synth.NVFP4, sfmt=sfmt, I_sh=I_sh, bias="zipf:1.0",
                            act_fmt=synth.ACT_NVFP4, swiglu_limit=limit)
    inp = synth.make_inputs(sh, seed=seed, pool_rows=2048)
    inp = synth.vary_globals(inp, seed + 1)
    d = staging.to_device(inp, DEV)
    rt = moe.Routing(M, E, k, DEV)
    moe.route_topk(rt, x=d.x, w_router=d.Wr, bias=d.bias, routed_scale=sh.routed_scale,
                   logits_out=torch.empty((M, E), dtype=torch.float32, device=DEV))
    xqp = torch.empty((M * k, H // 2), dtype=torch.uint8, device=DEV)
    xsp = torch.empty((M * k, H // 16), dtype=torch.uint8, device=DEV)
    moe.quant_act_nvfp4(d.x, inp.x_gscale, xqp, xsp, routing=rt)
    return sh, inp, d, rt, xqp, xsp


def _h4_compare(ghq, ghs, rows_h, hg):
    """h bytes against the oracle's NVFP4 requant of its own fp64 h (read in
    fp32): codes equal but at rounding midpoints of fp32 vs fp64 sums."""
    eq, tot, worst = 0, 0, 0.0
    for b, (h, g) in enumerate(zip(rows_h, hg)):
        rq, rs = orc.nvfp4_quant_f32(h[None, :].astype(np.float32), g)
        eq += int(np.sum(rq[0] == ghq[b])) + int(np.sum(rs[0] == ghs[b]))
        tot += rq.shape[1] + rs.shape[1]
        hd = orc.nvfp4_dequant(ghq[b:b + 1], ghs[b:b + 1], g)[0]
        worst = max(worst, rel_l2(hd, orc.nvfp4_dequant(rq, rs, g)[0]))
    return eq / tot, worst


@pytest.mark.parametrize("H,I,limit", [(512, 256, 0.0), (2560, 256, 0.0), (2560, 768, 0.5)])
def test_gate_up_down_nvfp4a_routed_parity(H, I, limit):
    """W4A4 routed experts: gate_up on NVFP4 activations writes NVFP4 h with
    each expert's global; down reads it (I = 256: along the rows; 768: along K)."""
    M, E, k = 40, 6, 3
    sh, inp, d, rt, xqp, xsp = _a4_setup(M, H, E, k, I, seed=21, limit=limit)
    P = M * k
    hq = torch.empty((P, I // 2), dtype=torch.uint8, device=DEV)
    hs = torch.empty((P, I // 16), dtype=torch.uint8, device=DEV)
    moe.expert_gate_up_nvfp4a(d.w13, M, H, I, E, k, xqp, xsp, inp.x_gscale, d.h_globals, hq, hs, routing=rt,
                              swiglu_limit=limit)
    y = torch.full((P, H), float("nan"), dtype=torch.float32, device=DEV)
    moe.expert_down_nvfp4a(d.w2, M, H, I, E, k, hq, hs, d.h_globals, y, routing=rt)
    torch.cuda.synchronize()
    bucket, ids = np_of(rt.bucket), np_of(rt.topk_ids).ravel()
    xq, xs = orc.nvfp4_quant_bf16(inp.x, inp.x_gscale)
    a = orc.nvfp4_dequant(xq, xs, inp.x_gscale)
    hs_ref, hgs = [], []
    for b in range(P):
        p = bucket[b]
        m13 = inp.w13.expert(ids[p])
        hs_ref.append(orc.gate_up(orc.Mat(m13.fmt, m13.packed, m13.scales, m13.gscale), H, I, a[p // k], limit))
        hgs.append(float(inp.h_gscale[ids[p]]))
    frac, worst = _h4_compare(np_of(hq), np_of(hs), hs_ref, hgs)
    assert frac >= 0.999, frac
    assert worst < 0.1, worst   # a flipped code is one E2M1 step (up to 1/3 of the value)
    gy = np_of(y)
    worst_y = 0.0
    for b in range(P):
        p = bucket[b]
        m2 = inp.w2.expert(ids[p])
        hd = orc.nvfp4_dequant(np_of(hq)[b:b + 1], np_of(hs)[b:b + 1], float(inp.h_gscale[ids[p]]))[0]
        yr = orc.down(orc.Mat(m2.fmt, m2.packed, m2.scales, m2.gscale), H, I, hd)
        worst_y = max(worst_y, rel_l2(gy[p], yr))
    assert worst_y < 2e-3, worst_y


@pytest.mark.parametrize("M", [23, 70])
def test_dense_nvfp4a_expert_parity(M):
    """The NVFP4 shared expert on NVFP4 activations (one expert over all rows)."""
    H, I = 384, 256
    sh, inp, d, rt, _, _ = _a4_setup(M, H, 4, 2, 128, seed=23, I_sh=I, sfmt=synth.NVFP4)
    xq = torch.empty((M, H // 2), dtype=torch.uint8, device=DEV)
    xs = torch.empty((M, H // 16), dtype=torch.uint8, device=DEV)
    moe.quant_act_nvfp4(d.x, inp.x_gscale, xq, xs)
    hq = torch.empty((M, I // 2), dtype=torch.uint8, device=DEV)
    hs = torch.empty((M, I // 16), dtype=torch.uint8, device=DEV)
    moe.expert_gate_up_nvfp4a(d.sh13, M, H, I, 1, 1, xq, xs, inp.x_gscale, d.sh_h_global, hq, hs)
    y = torch.empty((M, H), dtype=torch.float32, device=DEV)
    moe.expert_down_nvfp4a(d.sh2, M, H, I, 1, 1, hq, hs, d.sh_h_global, y)
    torch.cuda.synchronize()
    a = orc.nvfp4_dequant(np_of(xq), np_of(xs), inp.x_gscale)
    m13, m2 = orc.Mat.from_synth(inp.sh13), orc.Mat.from_synth(inp.sh2)
    frac, _ = _h4_compare(np_of(hq), np_of(hs), [orc.gate_up(m13, H, I, a[r]) for r in range(M)],
                          [inp.sh_h_gscale] * M)
    assert frac >= 0.999, frac
    gy = np_of(y)
    for r in range(M):
        hd = orc.nvfp4_dequant(np_of(hq)[r:r + 1], np_of(hs)[r:r + 1], inp.sh_h_gscale)[0]
        assert rel_l2(gy[r], orc.down(m2, H, I, hd)) < 2e-3
