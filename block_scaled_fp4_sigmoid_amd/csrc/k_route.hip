// k_route.hip — router GEMV, sigmoid top-k with renormalized weights, and the
// route step that groups each expert's rows into 8-row tiles (gfx950).
//
// Pages: sgl-nvidia-mega PR #24, "Modifications / Target spec" (one expert
// group, sigmoid scores, renormalized top-k); SGLang-NVIDIA-Mega README,
// DeepSeek-V4.1 slot table, rows "Router top-k" (one CTA per row) and "Routed
// experts (moe)" (8-row tiles; an expert with more than 8 rows takes several).
#include "dense_bf16_dev.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "quant_dev.h"
#include "route_dev.h"

#include <algorithm>

namespace moe {

// ---------------------------------------------------------------------------
// Router GEMV on the matrix cores.  x is bf16 and w_router fp32; w is split
// exactly into three bf16 pieces (w = w1 + w2 + w3: truncation keeps the top 8
// significant bits, the remainder is exact in fp32 and splits again), so every
// product x*wi is exact and the bf16 MFMA's fp32 accumulation gives the fp32
// dot product.  Units (one wave each) are (16-expert tile, K chunk, 64-row
// group); each writes partial logits for its K chunk, which the top-k step
// sums in chunk order (deterministic, no atomics).

#ifndef MOE_ROUTER_UNITS
#define MOE_ROUTER_UNITS 1024  // router waves to aim for: 16-expert tiles x K splits x row groups
#endif
#ifndef MOE_ROUTER_NBT
#define MOE_ROUTER_NBT 4  // 16-row blocks per router wave above 16 rows
#endif
constexpr int kRouterNBT = MOE_ROUTER_NBT;

RouterPlan router_plan(int M, int H, int E) {
    const int et = (E + 15) / 16;
    const int rg = M <= 16 ? 1 : (M + 16 * kRouterNBT - 1) / (16 * kRouterNBT);  // row groups of the waves
    const int nsteps = H / 128;  // chunks are whole multiples of 4 K-steps of 32
    const int want = std::max(1, MOE_ROUTER_UNITS / (et * rg));
    int splits = 1;
    for (int d = 1; d <= nsteps; ++d)
        if (nsteps % d == 0 && d <= want && d <= 32) splits = d;
    return RouterPlan{splits, H / splits, rg, M <= 16 && splits > 1 ? (splits + 3) & ~3 : 0};
}

__device__ __forceinline__ void split3(float w, uint32_t& b1, uint32_t& b2, uint32_t& b3) {
    const uint32_t u = __float_as_uint(w);
    const float w1 = __uint_as_float(u & 0xffff0000u);
    const float r = w - w1;
    const uint32_t ur = __float_as_uint(r);
    const float w2 = __uint_as_float(ur & 0xffff0000u);
    const float w3 = r - w2;
    b1 = u >> 16;
    b2 = ur >> 16;
    b3 = __float_as_uint(w3) >> 16;
}

// U: K-steps of 32 per round of loads (two rounds in flight); NBT: 16-row
// blocks of the row group (1 when M <= 16).  XS: the four waves of a
// workgroup (four 16-expert tiles of the same K chunk and row group) share
// each round's x tile through LDS instead of each loading it.
template <int U, int NBT, bool XS>
__global__ __launch_bounds__(256) void k_router_partials(const uint16_t* __restrict__ x,
                                                         const float* __restrict__ w_router,
                                                         int M, int H, int E, int splits, int sp,
                                                         int kchunk, int units, int nmain,
                                                         float* __restrict__ partials, int nquant,
                                                         uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                         float xg4, Bf16Side side, int stage) {
    // a bf16 shared-expert stage riding along: after the router and quant
    // workgroups, or first when the grid exceeds two workgroups per CU (placed
    // last it then ran in the launch's tail: skew 200.8 -> 198.7 us per step)
    const int nside = (int)gridDim.x - nmain - nquant;
    const bool side_first = (int)gridDim.x > 512;
    const int sb = side_first ? (int)blockIdx.x : (int)blockIdx.x - nmain - nquant;
    if (sb >= 0 && sb < nside) {
        bf16_side_block(side, stage, sb);
        return;
    }
    const int bx = side_first ? (int)blockIdx.x - nside : (int)blockIdx.x;
    if (bx >= nmain) {  // x in token order: MXFP8 (256 blocks of 32 values), or
        const int b = (bx - nmain) * 256 + threadIdx.x;  // NVFP4 with global xg4 > 0 (of 16)
        if (xg4 > 0.0f) {
            if (b < M * (H / 16)) quant_nvfp4_bf16x16(x + (size_t)b * 16, xg4, xq + (size_t)b * 8, xs + b);
        } else if (b < M * (H / 32)) {
            quant_block32(x + (size_t)b * 32, xq + (size_t)b * 32, xs + b);
        }
        return;
    }
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int unit = bx * 4 + wave;
    if (!XS && unit >= units) return;  // XS: every workgroup is full (units a multiple of 4)
    const int et = (E + 15) / 16;
    const int te = unit % et;
    const int kc = (unit / et) % splits;
    const int rgi = unit / (et * splits);
    const int i = lane & 15, g = lane >> 4;
    const int e = te * 16 + i;
    const bool ev = e < E;
    const float* wrow = w_router + (size_t)(ev ? e : 0) * H;
    const int r0 = rgi * 16 * NBT;
    const int nb = min(NBT, (M - r0 + 15) / 16);
    const uint16_t* xr[NBT];
    bool xv[NBT];
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
        const int r = r0 + j * 16 + i;
        xv[j] = (j < nb) && (r < M);
        xr[j] = x + (size_t)(xv[j] ? r : 0) * H;
    }
    v4f acc[NBT];
#pragma unroll
    for (int j = 0; j < NBT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

    // K rounds of U steps of 32, software-pipelined over two buffers: the
    // loads of round r + 1 are in flight while round r's MFMAs run.  The
    // chunk holds an even number of rounds (the launch picks U so that 64 U
    // divides kchunk), and every load is unconditional: lanes past E or rows
    // past M read row 0 and are zeroed by a select, so no branch separates an
    // MFMA from the read of its accumulator.
    // XS: the round's x tile, 16 NBT rows x 32 U values (bf16), rows padded by
    // 16 bytes: 64 NBT U chunks of 16 bytes, chunk c = (row c / (4 U), part
    // c % (4 U)), thread t loading chunks t, t + 256, ... (threads past the
    // last chunk load none)
    constexpr int kXRow = 64 * U + 16;  // bytes per tile row
    constexpr int kXTile = 16 * NBT * kXRow;
    constexpr int kXCh = 64 * NBT * U, kXN = (kXCh + 255) / 256;
    __shared__ __align__(16) uint8_t sx[XS ? 2 * kXTile : 16];
    const uint16_t* xrt[kXN];
    int xso[kXN];
    bool xct[kXN];
#pragma unroll
    for (int n = 0; n < kXN; ++n) {
        const int c = threadIdx.x + 256 * n;
        const int row = c / (4 * U), part = c % (4 * U);
        const int r = r0 + row;
        xct[n] = XS && c < kXCh;
        xrt[n] = x + (size_t)(r < M ? r : 0) * H + 8 * part;
        xso[n] = row * kXRow + 16 * part;
    }
    struct Round {
        float4 wl[U][2];
        v4i xb[U][NBT];  // the lane's B operands (each wave loads them), or
        v4i xt[kXN];     // the thread's chunks of the x tile (XS)
    };
    auto load = [&](int k0, Round& R) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + 32 * u + 8 * g;
            R.wl[u][0] = *reinterpret_cast<const float4*>(wrow + kk);
            R.wl[u][1] = *reinterpret_cast<const float4*>(wrow + kk + 4);
            if constexpr (!XS) {
#pragma unroll
                for (int j = 0; j < NBT; ++j) R.xb[u][j] = load16(xr[j] + kk);
            }
        }
        if constexpr (XS) {
#pragma unroll
            for (int n = 0; n < kXN; ++n)
                if (kXCh % 256 == 0 || xct[n]) R.xt[n] = load16(xrt[n] + k0);
        }
    };
    // XS: the tile of a round into LDS buffer b (rows past M hold row 0's
    // values; the MFMA inputs of those rows are zeroed below)
    auto tile_store = [&](const Round& R, int b) {
        if constexpr (XS) {
#pragma unroll
            for (int n = 0; n < kXN; ++n)
                if (kXCh % 256 == 0 || xct[n]) *reinterpret_cast<v4i*>(sx + b * kXTile + xso[n]) = R.xt[n];
        }
    };
    auto tile_read = [&](Round& R, int b) {
        if constexpr (XS) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < NBT; ++j)
                    R.xb[u][j] =
                        *reinterpret_cast<const v4i*>(sx + b * kXTile + (16 * j + i) * kXRow + 64 * u + 16 * g);
        }
    };
    auto compute = [&](const Round& R) {
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float4 w0 = ev ? R.wl[u][0] : z, w1 = ev ? R.wl[u][1] : z;
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            uint32_t p1[4], p2[4], p3[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t a1, a2, a3, c1, c2, c3;
                split3(wv[2 * t], a1, a2, a3);
                split3(wv[2 * t + 1], c1, c2, c3);
                p1[t] = a1 | (c1 << 16);
                p2[t] = a2 | (c2 << 16);
                p3[t] = a3 | (c3 << 16);
            }
            const v8bf A1 = __builtin_bit_cast(v8bf, v4i{(int)p1[0], (int)p1[1], (int)p1[2], (int)p1[3]});
            const v8bf A2 = __builtin_bit_cast(v8bf, v4i{(int)p2[0], (int)p2[1], (int)p2[2], (int)p2[3]});
            const v8bf A3 = __builtin_bit_cast(v8bf, v4i{(int)p3[0], (int)p3[1], (int)p3[2], (int)p3[3]});
            // every block runs its MFMAs (blocks past the rows multiply zeros)
#pragma unroll
            for (int j = 0; j < NBT; ++j) {
                const v8bf b = __builtin_bit_cast(v8bf, (j < nb && xv[j]) ? R.xb[u][j] : v4i{0, 0, 0, 0});
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, b, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, b, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A3, b, acc[j], 0, 0, 0);
            }
        }
    };
    const int kbeg = kc * kchunk, kend = kbeg + kchunk;
    constexpr int KR = 32 * U;  // K per round
    Round RA, RB;
    load(kbeg, RA);
    // (scheduling barriers keep each round's loads behind the previous
    // round's, so a round's MFMAs wait only for their own loads; the last
    // pair of rounds is peeled, so no load is issued past the chunk.  XS:
    // round A's tile sits in LDS buffer 0, round B's in buffer 1; a tile is
    // stored after the other buffer's round was read, one barrier each)
    if constexpr (XS) {
        tile_store(RA, 0);
        __syncthreads();
    }
    int k0 = kbeg;
    for (; k0 + 2 * KR < kend; k0 += 2 * KR) {
        __builtin_amdgcn_sched_barrier(0);
        load(k0 + KR, RB);
        __builtin_amdgcn_sched_barrier(0);
        tile_read(RA, 0);
        compute(RA);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (XS) {
            tile_store(RB, 1);
            __syncthreads();
        }
        load(k0 + 2 * KR, RA);
        __builtin_amdgcn_sched_barrier(0);
        tile_read(RB, 1);
        compute(RB);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (XS) {
            tile_store(RA, 0);
            __syncthreads();
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    load(k0 + KR, RB);
    __builtin_amdgcn_sched_barrier(0);
    tile_read(RA, 0);
    compute(RA);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XS) {
        tile_store(RB, 1);
        __syncthreads();
    }
    tile_read(RB, 1);
    compute(RB);
    __builtin_amdgcn_sched_barrier(0);
    // lane holds D[4g + t][i]: expert te*16 + 4g + t, row r0 + 16j + i; stores
    // of rows past M or experts past E go to an offset past the buffer (dropped).
    // Layout [splits][M][E], or [M][E][sp] (sp > 0)
    const uint32_t nsl = (uint32_t)(sp ? sp : splits);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(partials, nsl * (uint32_t)M * (uint32_t)E * 4u);
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
        const int r = r0 + j * 16 + i;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int ee = te * 16 + 4 * g + t;
            const uint32_t at = sp ? ((uint32_t)r * E + ee) * (uint32_t)sp + kc : ((uint32_t)kc * M + r) * E + ee;
            const uint32_t off = (j < nb && r < M && ee < E) ? at * 4u : kOOB;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][t]), rp, off, 0, 0);
        }
    }
}

hipError_t launch_router_partials(const uint16_t* x, const float* w_router, int M, int H, int E,
                                  const RouterPlan& plan, float* partials, uint8_t* xq, uint8_t* xs,
                                  const Bf16Side& side1, int stage1, hipStream_t stream, float xg4) {
    const int units = ((E + 15) / 16) * plan.splits * plan.row_groups;
    const int blocks = (units + 3) / 4;
    const int nquant = xq ? (M * (H / (xg4 > 0.0f ? 16 : 32)) + 255) / 256 : 0;
    const int extra = stage1 == kBf16None ? 0 : side1.blocks;
    const dim3 g(blocks + nquant + extra), b(256);
    // rounds of 128 K when a chunk holds pairs of them, else of 64 K (chunks
    // are multiples of 128); four row blocks take rounds of 64 K (registers)
    if (plan.kchunk % 128 != 0) return hipErrorInvalidValue;
    const bool wide = plan.kchunk % 256 == 0, one = M <= 16;
    // the four waves of a workgroup share an x tile when they hold four expert
    // tiles of one K chunk and row group: E a multiple of 64
    const bool share = ((E + 15) / 16) % 4 == 0;
    auto run = [&](auto kern) {
        hipLaunchKernelGGL(kern, g, b, 0, stream, x, w_router, M, H, E, plan.splits, plan.sp, plan.kchunk, units,
                           blocks, partials, nquant, xq, xs, xg4, side1, stage1);
    };
    if (wide && one)
        share ? run(k_router_partials<4, 1, true>) : run(k_router_partials<4, 1, false>);
    else if (one)
        share ? run(k_router_partials<2, 1, true>) : run(k_router_partials<2, 1, false>);
    else
        share ? run(k_router_partials<2, kRouterNBT, true>) : run(k_router_partials<2, kRouterNBT, false>);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k: one workgroup per row (the pages' one CTA per row).  Scores are fp64
// sigmoids of the fp32 logits; keys add the optional selection bias; the
// order is key descending, then expert ascending.


// fp64 key -> unsigned integer with the same order (+0 and -0 equal).
__device__ __forceinline__ uint64_t ordered_key(double v) {
    if (v == 0.0) v = 0.0;
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// A candidate: order-preserving key and expert id.  Better = larger key, then
// smaller id (the expert order among equal scores).  Branch-free, so the
// selection below runs without divergence.
struct Cand {
    uint64_t key;
    int id;
};
__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
    return (a.key > b.key) | ((a.key == b.key) & (a.id < b.id));
}
__device__ __forceinline__ void take_if(Cand& dst, const Cand& src, bool c) {
    dst.key = c ? src.key : dst.key;
    dst.id = c ? src.id : dst.id;
}

// Wave-wide max / min of a 32-bit value, returned uniform.  Inside each row
// of 16 lanes four DPP exchanges (pair swap, quad half swap, half-row mirror,
// row mirror) leave the row's result in every lane of the row; two row
// broadcasts then carry it to lane 63 (rows 1 and 3 take lane 15 of the row
// before them, rows 2 and 3 take lane 31).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
    // lanes a move does not write take the identity (0 for max, ~0 for min),
    // so each move folds into the max / min as one DPP instruction
    constexpr int id = MAX ? 0 : -1;
    auto step = [](uint32_t a, int b) { return MAX ? max(a, (uint32_t)b) : min(a, (uint32_t)b); };
    v = step(v, __builtin_amdgcn_update_dpp(id, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v = step(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v = step(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = step(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = step(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = step(v, __builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The lane holding the wave's best candidate (larger key, then smaller id),
// uniform.  The high key words decide almost always: the max of the high
// words, and the low words (then the ids) only among the lanes tied on it.
__device__ __forceinline__ int wave_best_lane(const Cand& c) {
    const uint32_t hi = (uint32_t)(c.key >> 32), lo = (uint32_t)c.key;
    const uint32_t H = wave_reduce_u32<true>(hi);
    uint64_t tied = __ballot(hi == H);
    if (__popcll(tied) > 1) {  // uniform
        const uint32_t L = wave_reduce_u32<true>(hi == H ? lo : 0u);
        tied = __ballot(hi == H && lo == L);
        if (__popcll(tied) > 1) {
            const uint32_t id = wave_reduce_u32<false>((hi == H && lo == L) ? (uint32_t)c.id : 0xffffffffu);
            tied = __ballot(hi == H && lo == L && (uint32_t)c.id == id);
        }
    }
    return __ffsll((unsigned long long)tied) - 1;
}

// Top-k of one row by wave 0: lane l holds experts l + 64t (t < KT) sorted
// best first (a bitonic network in registers), then k rounds of a wave-wide
// arg-max over the list heads; the winning lane drops its head.  Experts
// past E carry key 0, below every score.  Returns, in lane j < k, the j-th
// chosen expert.
template <int KT>
__device__ int select_topk(const uint64_t* s_ord, int E, int k, int lane) {
    Cand c[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int e = lane + 64 * t;
        c[t].key = e < E ? s_ord[e] : 0;
        c[t].id = e;
    }
#pragma unroll
    for (int size = 2; size <= KT; size <<= 1)
#pragma unroll
        for (int stride = size / 2; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < KT; ++i) {
                const int j = i ^ stride;
                if (j <= i) continue;
                // (i & size) == 0: this pair ends best-first
                const bool swap = ((i & size) == 0) ? better(c[j], c[i]) : better(c[i], c[j]);
                const Cand ci = c[i];
                take_if(c[i], c[j], swap);
                take_if(c[j], ci, swap);
            }
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        const int wl = wave_best_lane(c[0]);
        const int wid = __builtin_amdgcn_readlane(c[0].id, wl);
        const bool mine = wl == lane;
#pragma unroll
        for (int t = 0; t + 1 < KT; ++t) take_if(c[t], c[t + 1], mine);
        c[KT - 1].key = mine ? 0 : c[KT - 1].key;
        my_id = lane == j ? wid : my_id;
    }
    return my_id;
}

// Phases 2 and 3 of a row's top-k, by wave 0 (lane = its lane): the k slots
// picked from the keys in LDS, then the weights, the chosen scores summed in
// slot order.
__device__ __forceinline__ void topk_write_row(const uint64_t* s_ord, const double* s_sc, int r, int E, int k,
                                               float routed_scale, const moe_routing& route, int lane) {
    int my_id;
    if (E <= 256)
        my_id = select_topk<4>(s_ord, E, k, lane);
    else if (E <= 512)
        my_id = select_topk<8>(s_ord, E, k, lane);
    else
        my_id = select_topk<16>(s_ord, E, k, lane);
    const double my_sc = lane < k ? s_sc[my_id] : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
        const uint64_t b = __double_as_longlong(my_sc);
        const uint64_t v = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), j) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, j);
        sum += __longlong_as_double((long long)v);
    }
    if (lane < k) {
        route.topk_ids[(size_t)r * k + lane] = my_id;
        route.topk_w[(size_t)r * k + lane] = (float)(((double)routed_scale * my_sc) / sum);
    }
}

// The partial logits of expert e of row r, all in one round of loads
// (splits <= 32): 16-byte loads in the expert-contiguous layout (sp > 0), else
// split-major.
__device__ __forceinline__ void load_partials(const float* __restrict__ partials, int splits, int sp, int M, int E,
                                              int r, int e, float (&p)[32]) {
    if (sp) {
        const float* pe = partials + ((size_t)r * E + e) * sp;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 v = 4 * q < splits ? *reinterpret_cast<const float4*>(pe + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
            p[4 * q] = v.x;
            p[4 * q + 1] = v.y;
            p[4 * q + 2] = v.z;
            p[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < 32; ++u) p[u] = u < splits ? partials[((size_t)u * M + r) * E + e] : 0.f;
    }
}

// The logit (partials summed in chunk order), its fp64 score and key into LDS.
__device__ __forceinline__ void score_expert(const float (&p)[32], int splits, const float* __restrict__ bias,
                                             float* __restrict__ logits_out, int r, int E, int e, uint64_t* s_ord,
                                             double* s_sc) {
    float lg = p[0];
#pragma unroll
    for (int u = 1; u < 32; ++u)
        if (u < splits) lg = lg + p[u];
    if (logits_out) logits_out[(size_t)r * E + e] = lg;
    const double sc = 1.0 / (1.0 + exp(-(double)lg));
    s_sc[e] = sc;
    s_ord[e] = ordered_key(sc + (bias ? (double)bias[e] : 0.0));
}

// NE experts per thread and pass: 2 above 256 experts, so their partials
// arrive in one round of loads instead of one round per pass.
template <int NE>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ partials, int splits, int sp,
                                              const float* __restrict__ bias, int M, int E, int k,
                                              float routed_scale, float* __restrict__ logits_out,
                                              moe_routing route, Bf16Side side, int stage) {
    if ((int)blockIdx.x >= M) {  // a bf16 shared-expert stage riding along
        bf16_side_block(side, stage, blockIdx.x - M);
        return;
    }
    // Phase 1: every thread owns experts tid + 256q, sums their partial
    // logits in chunk order and stores the fp64 score and the order-preserving
    // integer form of the key in LDS.  Phase 2: wave 0 picks the k slots.
    // Phase 3: the weights, with the chosen scores summed in slot order.
    __shared__ uint64_t s_ord[kMaxE];
    __shared__ double s_sc[kMaxE];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256 * NE) {
        float p[NE][32];
#pragma unroll
        for (int n = 0; n < NE; ++n)
            if (e + 256 * n < E) load_partials(partials, splits, sp, M, E, r, e + 256 * n, p[n]);
#pragma unroll
        for (int n = 0; n < NE; ++n)
            if (e + 256 * n < E) score_expert(p[n], splits, bias, logits_out, r, E, e + 256 * n, s_ord, s_sc);
    }
    __syncthreads();
    if (tid < 64) topk_write_row(s_ord, s_sc, r, E, k, routed_scale, route, tid);
}

// Router and top-k of one row in one workgroup, for routers small enough
// that every row's workgroup reads all of W_r (E <= 64, E * H <= 32768: the
// partial logits, their launch boundary and the top-k launch go away).  The
// E2 = max(4, pow2(E)) expert slots of a row take T = 256 / E2 threads each;
// thread (e, part) takes the 8-value chunks part, part + T, ... of H (x and
// W_r rows read in 16- and 32-byte pieces), multiplies in fp64 (a bf16 x
// fp32 product is exact there) and adds in fp64; the T partial sums meet in a
// fixed butterfly, and the logit is their sum rounded once to fp32.  Blocks
// past M quantize x in token order, as the router launch's quant blocks do.
__global__ __launch_bounds__(256) void k_router_topk_row(const uint16_t* __restrict__ x,
                                                         const float* __restrict__ w_router,
                                                         const float* __restrict__ bias, int M, int H, int E,
                                                         int k, float routed_scale, float* __restrict__ logits_out,
                                                         moe_routing route, uint8_t* __restrict__ xq,
                                                         uint8_t* __restrict__ xs, float xg4) {
    if ((int)blockIdx.x >= M) {
        const int b = ((int)blockIdx.x - M) * 256 + threadIdx.x;
        if (xg4 > 0.0f) {
            if (b < M * (H / 16)) quant_nvfp4_bf16x16(x + (size_t)b * 16, xg4, xq + (size_t)b * 8, xs + b);
        } else if (b < M * (H / 32)) {
            quant_block32(x + (size_t)b * 32, xq + (size_t)b * 32, xs + b);
        }
        return;
    }
    __shared__ uint64_t s_ord[kSmallRouterE];
    __shared__ double s_sc[kSmallRouterE];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    int e2 = 4;
    while (e2 < E) e2 <<= 1;
    const int T = 256 / e2;  // a power of two, 4..64: a slot's threads sit in one wave
    const int e = tid / T, part = tid % T;
    const bool ev = e < E;
    const uint16_t* xr = x + (size_t)r * H;
    const float* wr = w_router + (size_t)(ev ? e : 0) * H;
    // kB chunks per round of loads (E * H <= 32768 gives at most 32 per
    // thread); chunks past H load chunk `part` again and are skipped; four
    // accumulators (value pair i of a chunk) added in a fixed order
    constexpr int kB = 8;
    const int nch = H / 8;
    double a[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c0 = part; c0 < nch; c0 += kB * T) {
        v4i xv[kB];
        float4 w0[kB], w1[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int c = c0 + u * T < nch ? c0 + u * T : part;
            xv[u] = load16(xr + 8 * c);
            w0[u] = *reinterpret_cast<const float4*>(wr + 8 * c);
            w1[u] = *reinterpret_cast<const float4*>(wr + 8 * c + 4);
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (c0 + u * T < nch) {
                const uint32_t xw[4] = {(uint32_t)xv[u].x, (uint32_t)xv[u].y, (uint32_t)xv[u].z, (uint32_t)xv[u].w};
                const float wv[8] = {w0[u].x, w0[u].y, w0[u].z, w0[u].w, w1[u].x, w1[u].y, w1[u].z, w1[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = fma((double)bf16_to_f32(xw[i] & 0xffffu), (double)wv[2 * i], a[i]);
                    a[i] = fma((double)bf16_to_f32(xw[i] >> 16), (double)wv[2 * i + 1], a[i]);
                }
            }
        }
    }
    double acc = (a[0] + a[1]) + (a[2] + a[3]);
    for (int off = 1; off < T; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (part == 0 && ev) {
        const float lg = (float)acc;
        if (logits_out) logits_out[(size_t)r * E + e] = lg;
        const double sc = 1.0 / (1.0 + exp(-(double)lg));
        s_sc[e] = sc;
        s_ord[e] = ordered_key(sc + (bias ? (double)bias[e] : 0.0));
    }
    __syncthreads();
    if (tid < 64) topk_write_row(s_ord, s_sc, r, E, k, routed_scale, route, tid);
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket(int M, int E, int k, moe_routing route, Bf16Side side,
                                                          int stage, int H, int2* yrec) {
    if (blockIdx.x > 0) {  // a bf16 shared-expert stage riding along
        bf16_side_block(side, stage, blockIdx.x - 1);
        return;
    }
    __shared__ __align__(16) uint8_t s_lds[kBucketLdsMax];
    bucket_step<kBucketThreads>(M, E, k, route, s_lds, H, yrec);
}

// The route step alone in its launch: one workgroup of 1024 threads, which
// places up to 384 rows in one chunk.
__global__ __launch_bounds__(kBucketThreadsBig) void k_bucket_big(int M, int E, int k, moe_routing route, int H,
                                                                 int2* yrec) {
    __shared__ __align__(16) uint8_t s_lds[kBucketLdsBig];
    bucket_step<kBucketThreadsBig>(M, E, k, route, s_lds, H, yrec);
}

hipError_t launch_topk(const float* partials, int splits, int sp, const float* bias, int M, int E, int k,
                       float routed_scale, float* logits_out, const moe_routing& route, const Bf16Side& side2,
                       int stage2, hipStream_t stream) {
    const int extra2 = stage2 == kBf16None ? 0 : side2.blocks;
    if (E > 256)
        hipLaunchKernelGGL(k_topk<2>, dim3(M + extra2), dim3(256), 0, stream, partials, splits, sp, bias, M, E, k,
                           routed_scale, logits_out, route, side2, stage2);
    else
        hipLaunchKernelGGL(k_topk<1>, dim3(M + extra2), dim3(256), 0, stream, partials, splits, sp, bias, M, E, k,
                           routed_scale, logits_out, route, side2, stage2);
    return hipGetLastError();
}

hipError_t launch_topk_bucket(const float* partials, int splits, int sp, const float* bias, int M, int E,
                              int k, float routed_scale, float* logits_out,
                              const moe_routing& route, const Bf16Side& side2, int stage2,
                              const Bf16Side& side3, int stage3, hipStream_t stream, int H, int2* yrec) {
    hipError_t e = launch_topk(partials, splits, sp, bias, M, E, k, routed_scale, logits_out, route, side2, stage2,
                               stream);
    if (e != hipSuccess) return e;
    const int extra3 = stage3 == kBf16None ? 0 : side3.blocks;
    if (extra3 == 0)
        hipLaunchKernelGGL(k_bucket_big, dim3(1), dim3(kBucketThreadsBig), 0, stream, M, E, k, route, H, yrec);
    else
        hipLaunchKernelGGL(k_bucket, dim3(1 + extra3), dim3(kBucketThreads), 0, stream, M, E, k, route, side3,
                           stage3, H, yrec);
    return hipGetLastError();
}

bool small_router(int M, int H, int E) { return M <= kSmallRouterRows && E <= kSmallRouterE && E * H <= 32768; }

hipError_t launch_router_topk_row(const uint16_t* x, const float* w_router, const float* bias, int M, int H,
                                  int E, int k, float routed_scale, float* logits_out, const moe_routing& route,
                                  uint8_t* xq, uint8_t* xs, float xg4, hipStream_t stream) {
    if (!small_router(M, H, E) || H % 32 != 0) return hipErrorInvalidValue;
    const int nquant = xq ? (M * (H / (xg4 > 0.0f ? 16 : 32)) + 255) / 256 : 0;
    hipLaunchKernelGGL(k_router_topk_row, dim3(M + nquant), dim3(256), 0, stream, x, w_router, bias, M, H, E, k,
                       routed_scale, logits_out, route, xq, xs, xg4);
    return hipGetLastError();
}

hipError_t launch_bucket(int M, int E, int k, const moe_routing& route, hipStream_t stream, int H, int2* yrec) {
    hipLaunchKernelGGL(k_bucket_big, dim3(1), dim3(kBucketThreadsBig), 0, stream, M, E, k, route, H, yrec);
    return hipGetLastError();
}

}  // namespace moe
