"""CPU-side checks of the C ABI: the HIP library loads, exports every symbol
include/moe.h declares, and its host-side validation refuses bad arguments
before touching the GPU (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

from block_scaled_fp4_sigmoid_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="moe.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_mi355.so is not built (run __graft_entry__.build())")
    return moe.lib()


def test_every_declared_symbol_is_exported(L):
    declared = _declared()
    assert set(declared) == set(moe.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_probe_library_exports():
    from block_scaled_fp4_sigmoid_amd import probe
    if not os.path.exists(probe.LIB_PATH):
        pytest.fail("libmoe_probe_mi355.so is not built (run __graft_entry__.build())")
    declared = _declared("moe_probe.h")
    assert set(declared) == set(probe.EXPORTS)
    P = probe.lib()
    for name in declared:
        assert hasattr(P, name), name
    # refusals return before any HIP call
    assert P.moe_probe_stream_read(None, 1152, 1152, 0x1000, None) == 1
    assert P.moe_probe_stream_read(0x1000, 1152, 1152, None, None) == 1
    assert P.moe_probe_stream_read(0x1000, 1152, 100, 0x1000, None) == 1    # row not a multiple of 64
    assert P.moe_probe_stream_read(0x1000, 1000, 1152, 0x1000, None) == 1   # bytes not whole rows
    assert P.moe_probe_stream_read(0x1008, 1152, 1152, 0x1000, None) == 1   # misaligned
    assert P.moe_probe_stream_read(0x1000, 0, 1152, 0x1000, None) == 1


def test_version_and_status_strings(L):
    assert moe.abi_version() == 10
    for rc in range(5):
        assert len(moe.status_str(rc)) > 0
    assert "unknown" in moe.status_str(99)


def test_tile_capacity_bound():
    for M, E, k in [(4, 16, 4), (8, 256, 8), (384, 256, 8), (48, 512, 10), (1, 1, 1)]:
        P = M * k
        assert moe.tile_capacity(M, E, k) == (P + 7) // 8 + min(E, P)
    assert moe.tile_capacity(0, 4, 1) == 0


def test_workspace_sizes(L):
    assert L.moe_route_workspace_bytes(8, 7168, 256, 8) > 0
    assert L.moe_route_workspace_bytes(8, 100, 256, 8) == 0          # H % 128
    assert L.moe_route_workspace_bytes(8, 7168, 2048, 8) == 0        # E > 1024
    assert L.moe_route_workspace_bytes(8, 7168, 16, 17) == 0         # k > E
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_BF16, 8, 7168, 256, 1, 1, 1) > 0
    # FP4: a K split (few items) needs fp32 partials [splits][rows][2I]; one split needs none
    few = L.moe_gate_up_workspace_bytes(moe.MOE_FMT_MXFP4, 8, 7168, 256, 1, 1, 1)
    assert few > 0 and few % (8 * 2 * 256 * 4) == 0 and few % 256 == 0
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_NVFP4, 2, 7168, 256, 8, 2, 0) > 0    # 4 experts x 4 blocks
    # enough items for the GPU: one K split, no partials
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_MXFP4, 64, 512, 2048, 64, 8, 0) == 0
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_MXFP4, 8, 100, 256, 1, 1, 1) == 0   # H % 128
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_BF16, 8, 7168, 256, 256, 8, 0) == 0  # bf16 routed


def _desc(**over):
    d = dict(M=8, H=1024, E=16, k=4, I=512, I_sh=0, routed_scale=1.0, eps=1e-6,
             w_router=0x1000, router_bias=None,
             w13=moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None),
             w2=moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None),
             sh13=moe.moe_weights(0, None, None, None), sh2=moe.moe_weights(0, None, None, None),
             gamma=0x1000)
    d.update(over)
    return moe.moe_layer_desc(**d)


def test_layer_desc_validation(L):
    ok = _desc()
    assert L.moe_layer_workspace_bytes(C.byref(ok)) > 0
    bad = [
        _desc(H=1000),                                   # H % 128
        _desc(I=500),                                    # I % 128
        _desc(k=0),
        _desc(k=17),                                     # k > E
        _desc(E=1025),
        _desc(M=5000),
        _desc(M=0),                                      # no rows
        _desc(H=16384 + 128),                            # H above 16384
        _desc(I=8192 + 128),                             # I above 8192
        _desc(w_router=None),
        _desc(gamma=None),
        _desc(w13=moe.moe_weights(moe.MOE_FMT_NVFP4, 0x1000, 0x1000, None)),  # NV without global
        _desc(w13=moe.moe_weights(moe.MOE_FMT_NVFP4, 0x1000, 0x1000, 0x1000)),  # w13/w2 formats differ
        _desc(I_sh=256, sh13=moe.moe_weights(moe.MOE_FMT_BF16, 0x1000, None, None)),  # sh13/sh2 differ
        _desc(I_sh=100, sh13=moe.moe_weights(moe.MOE_FMT_BF16, 0x1000, None, None),
              sh2=moe.moe_weights(moe.MOE_FMT_BF16, 0x1000, None, None)),
        _desc(w13=moe.moe_weights(moe.MOE_FMT_BF16, 0x1000, None, None),
              w2=moe.moe_weights(moe.MOE_FMT_BF16, 0x1000, None, None)),  # bf16 routed experts
        _desc(swiglu_limit=-0.5),
        _desc(swiglu_limit=float("nan")),
        _desc(act_fmt=2),                                # unknown activation format
        _desc(act_fmt=1, x_global=1.0, h_globals=0x1000),  # NVFP4 activations with MXFP4 experts
    ]
    nv = moe.moe_weights(moe.MOE_FMT_NVFP4, 0x1000, 0x1000, 0x1000)
    a4 = dict(w13=nv, w2=nv, act_fmt=1, x_global=0.01, h_globals=0x1000)
    assert L.moe_layer_workspace_bytes(C.byref(_desc(**a4))) > 0
    bad += [
        _desc(**dict(a4, x_global=0.0)),
        _desc(**dict(a4, x_global=float("inf"))),
        _desc(**dict(a4, h_globals=None)),
        _desc(**dict(a4, I_sh=256, sh13=nv, sh2=nv)),    # NVFP4 shared expert without its h global
        _desc(**dict(a4, I_sh=256, sh13=moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None),
                     sh2=moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None))),  # MXFP4 shared
    ]
    for d in bad:
        assert L.moe_layer_workspace_bytes(C.byref(d)) == 0


def test_calls_refuse_before_enqueueing(L):
    """Every refusal returns before any HIP call, so these run without a GPU."""
    d = _desc()
    rc = L.moe_layer(C.byref(d), None, None, None, None, None, None, None, None, 0, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = L.moe_layer(C.byref(d), 0x1000, 0x1000, 0x1000, None, None, None, None, None, 0, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    rc = L.moe_layer(C.byref(d), 0x1000, 0x1000, 0x1000, None, None, None, None, 0x1010, 1 << 30, None)
    assert rc == moe.MOE_ERR_WORKSPACE                     # misaligned
    rc = L.moe_layer(C.byref(d), 0x1000, 0x1000, 0x1000, None, None, None, None, 0x1000, 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE                     # too small
    # the MXFP8 next-input outputs come as a pair
    rc = L.moe_layer_mxfp8_out(C.byref(d), 0x1000, 0x1000, 0x1000, None, 0x1000, None, None, None, None,
                               0x1000, 1 << 30, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = L.moe_layer_mxfp8_out(C.byref(d), 0x1000, 0x1000, 0x1000, None, None, None, None, None, None,
                               0x1000, 16, None)
    assert rc == moe.MOE_ERR_WORKSPACE
    fin = [0x1000, 0x1000, None, 0x1000, 0x1000, 1e-6, 4, 256, 2, 0x1000, None]
    assert L.moe_finalize_rmsnorm_mxfp8(*fin, None, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_finalize_rmsnorm_mxfp8(*fin[:7], 200, *fin[8:], 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_finalize_rmsnorm_mxfp8(*fin[:5], -1.0, *fin[6:], 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act_mxfp8(None, 4, 64, None, 0, 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act_mxfp8(0x1000, 4, 48, None, 0, 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    # NVFP4 activations: the global must be positive and finite
    for g in (0.0, -1.0, float("nan"), float("inf")):
        assert L.moe_quant_act_nvfp4(0x1000, 4, 64, g, None, 0, 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act_nvfp4(0x1000, 4, 48, 1.0, None, 0, 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_act_nvfp4(None, 4, 64, 1.0, None, 0, 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    r = moe.moe_routing()  # bucket missing
    assert L.moe_quant_act_mxfp8(0x1000, 4, 64, C.byref(r), 2, 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    r.bucket = 0x1000
    assert L.moe_quant_act_mxfp8(0x1000, 4, 64, C.byref(r), 33, 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    # packing: format, shape and pointer checks
    assert L.moe_packed_scale_bytes(moe.MOE_FMT_MXFP4, 2, 32, 640) == 2 * 2 * 2 * 64 * 4
    assert L.moe_packed_scale_bytes(moe.MOE_FMT_NVFP4, 1, 16, 128) == 64 * 8
    assert L.moe_packed_scale_bytes(moe.MOE_FMT_MXFP4, 1, 24, 128) == 0     # N % 16
    assert L.moe_packed_scale_bytes(moe.MOE_FMT_BF16, 1, 16, 128) == 0
    assert L.moe_pack_fp4(moe.MOE_FMT_BF16, 1, 16, 128, 0x1000, 0x1000, 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_fp4(moe.MOE_FMT_MXFP4, 1, 16, 100, 0x1000, 0x1000, 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_fp4(moe.MOE_FMT_MXFP4, 1, 16, 192, 0x1000, 0x1000, 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_fp4(moe.MOE_FMT_MXFP4, 1, 16, 128, None, 0x1000, 0x1000, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    r = moe.moe_routing(*([0x1000] * 10))
    # both x and logits_in, or neither
    assert L.moe_route_topk(None, None, None, None, 4, 128, 8, 2, 1.0, None, C.byref(r), 0x1000,
                            1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(0x1000, 0x1000, 0x1000, None, 4, 128, 8, 2, 1.0, 0x1000, C.byref(r),
                            0x1000, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    # x without logits_out
    assert L.moe_route_topk(0x1000, None, 0x1000, None, 4, 128, 8, 2, 1.0, None, C.byref(r), 0x1000,
                            1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    r_bad = moe.moe_routing(*([0x1000] * 9 + [None]))
    assert L.moe_route_topk(None, 0x1000, None, None, 4, 128, 8, 2, 1.0, None, C.byref(r_bad),
                            0x1000, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    w = moe.moe_weights(moe.MOE_FMT_BF16, 0x1000, None, None)
    # bf16 weights are only supported densely (shared expert)
    assert L.moe_expert_gate_up(C.byref(w), None, None, 0x1000, C.byref(r), 4, 128, 128, 8, 2, 0.0, None,
                                None, 0x1000, 0x1000, 1 << 20, None) == moe.MOE_ERR_UNSUPPORTED
    # the clamped SwiGLU's limit: negative or NaN refused
    for bad in (-1.0, float("nan")):
        assert L.moe_expert_gate_up(C.byref(w), None, None, 0x1000, None, 4, 128, 128, 1, 1, bad, None,
                                    None, 0x1000, 0x1000, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_down(C.byref(w), None, None, 0x1000, None, 4, 128, 100, 1, 1, 0x1000,
                             None) == moe.MOE_ERR_UNSUPPORTED
    # token-order gate_up: routed FP4 experts only, every pointer given
    gut = lambda wt, rt, lim=0.0, a=0x1000: L.moe_expert_gate_up_tok(C.byref(wt), a, 0x1000, rt, 4, 128, 128, 8, 2,
                                                                     lim, 0x1000, 0x1000, 0x1000, 1 << 20, None)
    mx = moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None)
    assert gut(w, C.byref(r)) == moe.MOE_ERR_UNSUPPORTED          # bf16 weights
    assert gut(mx, None) == moe.MOE_ERR_INVALID_ARG               # no route
    assert gut(mx, C.byref(r), a=None) == moe.MOE_ERR_INVALID_ARG
    assert gut(mx, C.byref(r), lim=-1.0) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_gate_up_tok(C.byref(mx), 0x1000, 0x1000, C.byref(r), 4, 128, 100, 8, 2, 0.0, 0x1000,
                                    0x1000, 0x1000, 1 << 20, None) == moe.MOE_ERR_UNSUPPORTED  # I % 128
    assert L.moe_expert_gate_up_tok(C.byref(mx), 0x1000, 0x1000, C.byref(r_bad), 4, 128, 128, 8, 2, 0.0, 0x1000,
                                    0x1000, 0x1000, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG  # routing array missing
    # W4A4: NVFP4 weights only, a positive activation global, the h globals given
    mx = moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None)
    nvw = moe.moe_weights(moe.MOE_FMT_NVFP4, 0x1000, 0x1000, 0x1000)
    gu4 = lambda wt, g, hg: L.moe_expert_gate_up_nvfp4a(C.byref(wt), 0x1000, 0x1000, g, None, 4, 128, 128, 1, 1,
                                                         0.0, hg, 0x1000, 0x1000, None)
    assert gu4(mx, 1.0, 0x1000) == moe.MOE_ERR_UNSUPPORTED
    assert gu4(nvw, 0.0, 0x1000) == moe.MOE_ERR_INVALID_ARG
    assert gu4(nvw, 1.0, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_down_nvfp4a(C.byref(mx), 0x1000, 0x1000, 0x1000, None, 4, 128, 128, 1, 1, 0x1000,
                                    None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_down_nvfp4a(C.byref(nvw), 0x1000, 0x1000, None, None, 4, 128, 128, 1, 1, 0x1000,
                                    None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_finalize_rmsnorm(0x1000, 0x1000, None, 0x1000, 0x1000, -1.0, 4, 128, 2, 0x1000,
                                  None, None) == moe.MOE_ERR_INVALID_ARG


def test_pair_output_size_limit(L):
    """Routed calls whose fp32 per-pair output y [M*k, H] would reach 2 GiB are
    refused (the kernels address it with 32-bit buffer offsets); the largest
    accepted shapes sit just under the limit."""
    limit = (1 << 31) - (1 << 20)
    # M=4096, k=9, H=16384: 2.25 GiB of y -> refused; k=7 (1.75 GiB) accepted
    assert 4096 * 9 * 16384 * 4 > limit and 4096 * 7 * 16384 * 4 <= limit
    assert L.moe_layer_workspace_bytes(C.byref(_desc(M=4096, E=32, k=9, H=16384))) == 0
    assert L.moe_layer_workspace_bytes(C.byref(_desc(M=4096, E=32, k=16, H=16384))) == 0
    assert L.moe_layer_workspace_bytes(C.byref(_desc(M=4096, E=32, k=7, H=16384))) > 0
    d = _desc(M=4096, E=32, k=9, H=16384)
    rc = L.moe_layer(C.byref(d), 0x1000, 0x1000, 0x1000, None, None, None, None, 0x1000, 1 << 40, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    r = moe.moe_routing(*([0x1000] * 11))
    for fmt in (moe.MOE_FMT_MXFP4, moe.MOE_FMT_NVFP4):
        w = moe.moe_weights(fmt, 0x1000, 0x1000, 0x1000)
        assert L.moe_expert_down(C.byref(w), 0x1000, 0x1000, None, C.byref(r), 4096, 16384, 128, 32, 9,
                                 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
        assert L.moe_expert_gate_up(C.byref(w), 0x1000, 0x1000, None, C.byref(r), 4096, 16384, 128, 32, 9,
                                    0.0, 0x1000, 0x1000, None, 0x1000, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    nvw = moe.moe_weights(moe.MOE_FMT_NVFP4, 0x1000, 0x1000, 0x1000)
    assert L.moe_expert_gate_up_nvfp4a(C.byref(nvw), 0x1000, 0x1000, 1.0, C.byref(r), 4096, 16384, 128, 32, 9,
                                       0.0, 0x1000, 0x1000, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_down_nvfp4a(C.byref(nvw), 0x1000, 0x1000, 0x1000, C.byref(r), 4096, 16384, 128, 32, 9,
                                    0x1000, None) == moe.MOE_ERR_UNSUPPORTED


def test_noalloc_refusals(L):
    """moe_layer_noalloc refuses, before any HIP call, an invalid description,
    missing pointers, and a layer whose workspace exceeds its static scratch."""
    assert L.moe_layer_noalloc(None, 0x1000, 0x1000, 0x1000, None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    d = _desc()
    assert L.moe_layer_noalloc(C.byref(d), None, 0x1000, 0x1000, None, None, None, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_noalloc(C.byref(_desc(H=1000)), 0x1000, 0x1000, 0x1000, None, None, None, None,
                               None) == moe.MOE_ERR_UNSUPPORTED
    # the 384-row step at hidden 7168, intermediate 2048 needs about 107 MiB of workspace
    wide = _desc(M=384, H=7168, E=256, k=8, I=2048)
    assert L.moe_layer_workspace_bytes(C.byref(wide)) > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_layer_noalloc(C.byref(wide), 0x1000, 0x1000, 0x1000, None, None, None, None,
                               None) == moe.MOE_ERR_SCRATCH
    assert b"static" in L.moe_status_str(moe.MOE_ERR_SCRATCH)
    # a 16-row decode-sized layer fits
    assert 0 < L.moe_layer_workspace_bytes(C.byref(_desc(M=16, H=7168, E=384, k=8, I=2048))) <= \
        moe.NOALLOC_SCRATCH_BYTES


def test_static_fp8_shared_refusals(L):
    """The static-FP8 shared expert: dense only, FP8S weights with their
    scale, finite positive static scales; in the layer description too."""
    f8 = moe.moe_weights(moe.MOE_FMT_FP8S, 0x1000, None, 0x1000)
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_FP8S, 7, 4096, 512, 1, 1, 1) > 0
    assert L.moe_gate_up_workspace_bytes(moe.MOE_FMT_FP8S, 7, 4096, 512, 64, 4, 0) == 0   # routed: no
    gu = lambda w, s_in, s_h, ws=0x1000: L.moe_expert_gate_up_fp8s(C.byref(w), 0x1000, s_in, s_h, 7, 4096, 512, 0.0,
                                                                   0x1000, ws, 1 << 30, None)
    mx = moe.moe_weights(moe.MOE_FMT_MXFP4, 0x1000, 0x1000, None)
    assert gu(mx, 0.1, 0.1) == moe.MOE_ERR_UNSUPPORTED
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert gu(f8, bad, 0.1) == moe.MOE_ERR_INVALID_ARG
        assert gu(f8, 0.1, bad) == moe.MOE_ERR_INVALID_ARG
        assert L.moe_expert_down_fp8s(C.byref(f8), 0x1000, bad, 7, 4096, 512, 0x1000, None) == moe.MOE_ERR_INVALID_ARG
    assert gu(moe.moe_weights(moe.MOE_FMT_FP8S, 0x1000, None, None), 0.1, 0.1) == moe.MOE_ERR_INVALID_ARG
    assert gu(f8, 0.1, 0.1, ws=0x1010) == moe.MOE_ERR_WORKSPACE
    assert L.moe_expert_down_fp8s(C.byref(mx), 0x1000, 0.1, 7, 4096, 512, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_down_fp8s(C.byref(f8), 0x1000, 0.1, 7, 4096, 500, 0x1000, None) == moe.MOE_ERR_UNSUPPORTED
    # FP8S routed experts are refused by the routed entry points
    r = moe.moe_routing(*([0x1000] * 11))
    assert L.moe_expert_down(C.byref(f8), 0x1000, 0x1000, None, C.byref(r), 4, 128, 128, 8, 2, 0x1000,
                             None) == moe.MOE_ERR_UNSUPPORTED
    ok = dict(I_sh=256, sh13=f8, sh2=f8, sh_in_scale=0.01, sh_h_scale=0.03)
    assert L.moe_layer_workspace_bytes(C.byref(_desc(**ok))) > 0
    nv = moe.moe_weights(moe.MOE_FMT_NVFP4, 0x1000, 0x1000, 0x1000)
    a4 = dict(w13=nv, w2=nv, act_fmt=1, x_global=0.01, h_globals=0x1000)
    assert L.moe_layer_workspace_bytes(C.byref(_desc(**dict(ok, **a4)))) > 0   # with NVFP4 activations
    for bad in (dict(ok, sh_in_scale=0.0), dict(ok, sh_h_scale=float("nan")),
                dict(ok, sh13=moe.moe_weights(moe.MOE_FMT_FP8S, 0x1000, None, None)),
                dict(ok, sh2=moe.moe_weights(moe.MOE_FMT_FP8S, None, None, 0x1000))):
        assert L.moe_layer_workspace_bytes(C.byref(_desc(**bad))) == 0
