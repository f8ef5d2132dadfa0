"""Pins of the oracle's router and route step: full sorts on small E,
top-k = all experts, renormalization sums, tie-breaks, bucket/tile
invariants, and logits against a numpy fp64 matmul."""
import numpy as np
import pytest

from block_scaled_fp4_sigmoid_amd import synth


def _keys(logits, bias):
    s = 1.0 / (1.0 + np.exp(-logits.astype(np.float64)))
    return s, s + (0.0 if bias is None else bias.astype(np.float64))


@pytest.mark.parametrize("E,k", [(1, 1), (5, 5), (8, 3), (16, 4), (64, 8), (300, 10)])
def test_topk_equals_full_sort(orc, E, k):
    rng = np.random.default_rng(E * 100 + k)
    for trial in range(20):
        l = (rng.standard_normal(E) * 2).astype(np.float32)
        bias = None if trial % 2 == 0 else (rng.standard_normal(E) * 0.05).astype(np.float32)
        scale = [1.0, 2.5][trial % 2]
        ids, w, s_sel = orc.topk_row(l, bias, k, scale)
        s, key = _keys(l, bias)
        order = np.lexsort((np.arange(E), -key))  # key desc, then id asc
        assert list(ids) == list(order[:k])
        assert np.allclose(s_sel, s[ids], rtol=4e-16, atol=0)  # libm vs numpy exp: <= 1 ulp
        # weights: unbiased scores renormalized over the chosen set, times scale
        ref = scale * s[ids] / s[ids].sum()
        assert np.allclose(w, ref, rtol=1e-7, atol=0)
        assert abs(float(np.sum(w.astype(np.float64))) - scale) <= 1e-6 * scale


def test_topk_all_experts_is_a_sorted_permutation(orc):
    rng = np.random.default_rng(7)
    E = 32
    l = rng.standard_normal(E).astype(np.float32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids, w, _ = orc.topk_row(l, b, E, 1.0)
    assert sorted(ids) == list(range(E))
    _, key = _keys(l, b)
    assert all(key[ids[i]] >= key[ids[i + 1]] for i in range(E - 1))


def test_single_expert_weight_is_scale(orc):
    ids, w, _ = orc.topk_row(np.array([0.3], np.float32), None, 1, 2.5)
    assert ids[0] == 0 and w[0] == np.float32(2.5)


def test_ties_go_to_lower_expert_id(orc):
    l = np.array([0.5, 1.0, 1.0, -2.0, 1.0, 0.5], np.float32)
    ids, _, _ = orc.topk_row(l, None, 4, 1.0)
    assert list(ids) == [1, 2, 4, 0]


def test_bias_only_selects(orc):
    """The bias moves experts into the top-k but the weights use the
    unbiased scores (a biased weight would differ)."""
    l = np.array([2.0, 0.0, 0.0, 0.0], np.float32)
    b = np.array([0.0, 0.0, 0.0, 1.0], np.float32)
    ids, w, _ = orc.topk_row(l, b, 2, 1.0)
    assert list(ids) == [3, 0]
    s = 1 / (1 + np.exp(-np.array([0.0, 2.0])))
    assert np.allclose(w, s / s.sum(), rtol=1e-7)


def test_route_buckets_and_tiles(orc):
    rng = np.random.default_rng(11)
    for M, E, k in [(1, 4, 2), (4, 16, 4), (48, 64, 6), (100, 8, 8), (384, 256, 8)]:
        logits = rng.standard_normal((M, E)).astype(np.float32)
        bias = (np.arange(E)[::-1] ** 1.5 / E).astype(np.float32)  # skew: low ids hot
        r = orc.route(logits, bias, k, 1.0)
        ids, off, bucket = r["ids"], r["offsets"], r["bucket"]
        P = M * k
        counts = np.bincount(ids.ravel(), minlength=E)
        assert off[0] == 0 and off[E] == P
        assert np.array_equal(np.diff(off), counts)
        assert sorted(bucket) == list(range(P))  # every pair once
        for e in range(E):
            ent = bucket[off[e]:off[e + 1]]
            assert all(ids.ravel()[p] == e for p in ent)
            rows = ent // k
            assert np.all(np.diff(rows) > 0)  # ascending rows, each row at most once
        # tiles: ceil(n/8) per expert, consecutive, (expert, tile) order
        nt = r["num_tiles"]
        assert nt == int(np.sum((counts + 7) // 8))
        assert nt <= orc.tile_capacity(M, E, k)
        te, tb, tr = r["tile_expert"], r["tile_begin"], r["tile_rows"]
        assert np.all(np.diff(te) >= 0)
        for t in range(nt):
            e = te[t]
            assert off[e] <= tb[t] < off[e + 1] and 1 <= tr[t] <= 8
            assert tb[t] + tr[t] <= off[e + 1]
            assert (tr[t] == 8) or (tb[t] + tr[t] == off[e + 1])
        covered = np.concatenate([np.arange(tb[t], tb[t] + tr[t]) for t in range(nt)])
        assert np.array_equal(covered, np.arange(P))


def test_route_matches_bruteforce_listing(orc):
    rng = np.random.default_rng(12)
    M, E, k = 9, 6, 3
    logits = rng.standard_normal((M, E)).astype(np.float32)
    r = orc.route(logits, None, k, 1.0)
    ids = r["ids"]
    ref = [r_ * k + j for e in range(E) for r_ in range(M) for j in range(k) if ids[r_, j] == e]
    assert list(r["bucket"]) == ref


def test_router_logits_vs_numpy(orc):
    rng = np.random.default_rng(13)
    M, H, E = 5, 256, 12
    x = synth._bf16_trunc(rng.standard_normal((M, H)).astype(np.float32))
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xv @ Wr.astype(np.float64).T
    got = orc.router_logits(x, Wr)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-12)


def test_zipf_workload_has_multi_tile_experts(orc):
    """The skewed workload's Zipf bias makes several experts take more than
    one 8-row tile (what that workload exists to exercise)."""
    inp = synth.make_inputs("skew-m48-h4096-e512-k10-nvfp4", seed=4, pool_rows=64)
    lg = orc.router_logits(inp.x, inp.Wr).astype(np.float32)
    r = orc.route(lg, inp.bias, inp.shape.k, inp.shape.routed_scale)
    counts = np.diff(r["offsets"])
    assert (counts > 8).sum() >= 3
