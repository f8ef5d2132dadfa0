// route_dev.h — the route step as a device function of one workgroup (of
// kBucketThreads threads, so it can run as an extra workgroup of a later
// launch, or of kBucketThreadsBig in a launch of its own; it reads only
// topk_ids).
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Routed
// experts (moe)": each expert's rows are grouped into tiles of at most 8 rows,
// an expert with more than 8 rows takes several tiles.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kBucketThreads = 256;
constexpr int kBucketThreadsBig = 1024;

// Exclusive scans of three arrays of kMaxE entries at once (kMaxE / NT per
// thread): each wave scans its lanes' sums with shuffles, and the wave totals
// (in scratch, 3 ints per wave) give each wave's base.  Two barriers.
template <int NT>
__device__ inline void block_exclusive_scan3(int* a, int* b, int* c, int* scratch, int& ta, int& tb, int& tc) {
    constexpr int EPT = kMaxE / NT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int va[EPT], vb[EPT], vc[EPT];
    int sa = 0, sb = 0, sc = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        va[i] = a[EPT * tid + i];
        vb[i] = b[EPT * tid + i];
        vc[i] = c[EPT * tid + i];
        sa += va[i];
        sb += vb[i];
        sc += vc[i];
    }
    int ia = sa, ib = sb, ic = sc;  // inclusive scans over the wave's lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int xa = __shfl_up(ia, off, 64), xb = __shfl_up(ib, off, 64), xc = __shfl_up(ic, off, 64);
        if (lane >= off) {
            ia += xa;
            ib += xb;
            ic += xc;
        }
    }
    if (lane == 63) {
        scratch[3 * w] = ia;
        scratch[3 * w + 1] = ib;
        scratch[3 * w + 2] = ic;
    }
    __syncthreads();
    int ba = 0, bb = 0, bc = 0;
    ta = tb = tc = 0;
#pragma unroll
    for (int v = 0; v < NT / 64; ++v) {
        const int wa = scratch[3 * v], wb = scratch[3 * v + 1], wc = scratch[3 * v + 2];
        if (v < w) {
            ba += wa;
            bb += wb;
            bc += wc;
        }
        ta += wa;
        tb += wb;
        tc += wc;
    }
    int ea = ba + ia - sa, eb = bb + ib - sb, ec = bc + ic - sc;  // exclusive bases of the thread's entries
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        a[EPT * tid + i] = ea;
        b[EPT * tid + i] = eb;
        c[EPT * tid + i] = ec;
        ea += va[i];
        eb += vb[i];
        ec += vc[i];
    }
    __syncthreads();
}

// Pairs per thread in one placement chunk, rows per chunk and bitmap words
// per expert of the route step of NT threads.  NT = 1024 places up to 384
// rows in one chunk (the 384-row step in one), with each word's count of
// earlier rows precomputed per expert so a rank costs two LDS reads; NT = 256
// places chunks of 128 rows and counts a rank's earlier words in a loop.
constexpr int kChunkPairsPerThread = 4;
template <int NT>
__host__ __device__ inline int bucket_chunk_rows(int k) {
    constexpr int cap = NT == kBucketThreadsBig ? 384 : 128;
    return cap < kChunkPairsPerThread * NT / k ? cap : kChunkPairsPerThread * NT / k;
}
template <int NT>
__host__ __device__ inline int bucket_words(int k) { return (bucket_chunk_rows<NT>(k) + 31) / 32; }

// LDS bytes the route step needs at most: five per-expert int arrays, the
// scan scratch, the placement bitmaps (and for NT = 1024 the per-word counts).
template <int NT>
constexpr size_t bucket_lds_max() {
    constexpr int W = (NT == kBucketThreadsBig ? 384 : 128) / 32;
    return (size_t)(5 * kMaxE + NT) * 4 + (size_t)kMaxE * W * 4 * (NT == kBucketThreadsBig ? 2 : 1);
}
constexpr size_t kBucketLdsMax = bucket_lds_max<kBucketThreads>();
constexpr size_t kBucketLdsBig = bucket_lds_max<kBucketThreadsBig>();

// ---------------------------------------------------------------------------
// Route step: one workgroup builds the expert buckets, 8-row tiles and the
// active-expert list from topk_ids (in a launch after the top-k one, so the
// ids written by the top-k workgroups are visible without a device-scope
// fence).  With yrec, also each pair's row of a grouped y of H columns
// (ygroup_rec).
template <int NT>
__device__ inline void bucket_step(int M, int E, int k, const moe_routing& route, uint8_t* lds, int H = 0,
                                   int2* yrec = nullptr) {
    const int tid = threadIdx.x;
    constexpr bool kBig = NT == kBucketThreadsBig;
    static_assert(!kBig || NT == kMaxE, "one expert per thread in the per-word counts");

    int* s_cnt = reinterpret_cast<int*>(lds);
    int* s_off = s_cnt + kMaxE;
    int* s_tile = s_off + kMaxE;
    int* s_act = s_tile + kMaxE;
    int* s_run = s_act + kMaxE;
    int* s_scan = s_run + kMaxE;
    uint32_t* s_bm = reinterpret_cast<uint32_t*>(s_scan + NT);  // E * bucket_words(k)
    const int P = M * k;
    const int R = bucket_chunk_rows<NT>(k);
    const int W = bucket_words<NT>(k);
    int* s_pre = reinterpret_cast<int*>(s_bm + E * W);  // kBig: earlier rows of the expert before each word
    for (int e = tid; e < kMaxE; e += NT) {
        s_cnt[e] = 0;
        s_run[e] = 0;
    }
    __syncthreads();
    // Pairs in placement chunks of R rows (R * k <= 4 * NT pairs: pairs
    // r0 * k + tid + NT q, q < 4).  The expert ids of a thread's pairs in the
    // first kIdChunks chunks stay in registers for the placement below.
    const int CP = R * k;  // pairs per chunk
    constexpr int kIdChunks = 4;
    int idr[kIdChunks][kChunkPairsPerThread];
#pragma unroll
    for (int ci = 0; ci < kIdChunks; ++ci)
#pragma unroll
        for (int q = 0; q < kChunkPairsPerThread; ++q) {
            const int pc = tid + NT * q;
            const int p = ci * CP + pc;
            idr[ci][q] = pc < CP && p < P ? route.topk_ids[p] : -1;
        }
#pragma unroll
    for (int ci = 0; ci < kIdChunks; ++ci)
#pragma unroll
        for (int q = 0; q < kChunkPairsPerThread; ++q)
            if (idr[ci][q] >= 0) atomicAdd(&s_cnt[idr[ci][q]], 1);
    for (int p = kIdChunks * CP + tid; p < P; p += NT) atomicAdd(&s_cnt[route.topk_ids[p]], 1);
    __syncthreads();
    for (int e = tid; e < kMaxE; e += NT) {
        const int c = s_cnt[e];
        s_off[e] = c;
        s_tile[e] = (c + 7) / 8;
        s_act[e] = c > 0 ? 1 : 0;
    }
    __syncthreads();
    int tot_pairs, tot_tiles, tot_act;
    block_exclusive_scan3<NT>(s_off, s_tile, s_act, s_scan, tot_pairs, tot_tiles, tot_act);
    for (int e = tid; e < E; e += NT) {
        const int c = s_cnt[e];
        route.expert_offsets[e] = s_off[e];
        if (c > 0) {
            route.active_experts[s_act[e]] = e;
            route.active_offsets[s_act[e]] = s_off[e];
        }
        for (int t = 0; 8 * t < c; ++t) {
            const int ti = s_tile[e] + t;
            route.tile_expert[ti] = e;
            route.tile_begin[ti] = s_off[e] + 8 * t;
            route.tile_rows[ti] = min(8, c - 8 * t);
        }
    }
    if (tid == 0) {
        route.expert_offsets[E] = P;
        *route.num_tiles = tot_tiles;
        *route.num_active = tot_act;
    }
    for (int sl = tot_act + tid; sl <= min(E, P); sl += NT) route.active_offsets[sl] = P;
    // Stable placement: chunks of R rows; a bitmap per expert marks the chunk's
    // rows that chose it, and a pair's rank within its expert is the number of
    // earlier rows (previous chunks + lower bits of this chunk's bitmap).
    for (int r0 = 0, ci = 0; r0 < M; r0 += R, ++ci) {
        for (int w = tid; w < E * W; w += NT) s_bm[w] = 0u;
        __syncthreads();
        int eq[kChunkPairsPerThread], rlq[kChunkPairsPerThread];
#pragma unroll
        for (int q = 0; q < kChunkPairsPerThread; ++q) {
            const int pc = tid + NT * q;
            const int p = r0 * k + pc;
            eq[q] = -1;
            rlq[q] = 0;
            if (pc < CP && p < P) {
                int ev = 0;
#pragma unroll
                for (int cj = 0; cj < kIdChunks; ++cj) ev = cj == ci ? idr[cj][q] : ev;  // registers, no dynamic index
                eq[q] = ci < kIdChunks ? ev : route.topk_ids[p];
                rlq[q] = p / k - r0;
                atomicOr(&s_bm[eq[q] * W + (rlq[q] >> 5)], 1u << (rlq[q] & 31));
            }
        }
        __syncthreads();
        int chunk_rows = 0;  // kBig: the chunk's rows of expert tid
        if constexpr (kBig) {
            if (tid < E) {
                for (int w = 0; w < W; ++w) {
                    s_pre[tid * W + w] = chunk_rows;
                    chunk_rows += __popc(s_bm[tid * W + w]);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < kChunkPairsPerThread; ++q) {
            if (eq[q] >= 0) {
                const int e = eq[q], rl = rlq[q];
                int rank = 0;
                if constexpr (kBig) {
                    rank = s_pre[e * W + (rl >> 5)];
                } else {
                    for (int w = 0; w < (rl >> 5); ++w) rank += __popc(s_bm[e * W + w]);
                }
                rank += __popc(s_bm[e * W + (rl >> 5)] & ((1u << (rl & 31)) - 1u));
                const int pair = r0 * k + tid + NT * q;
                route.bucket[s_off[e] + s_run[e] + rank] = pair;
                if (yrec) yrec[pair] = ygroup_rec(s_off[e], s_cnt[e], s_run[e] + rank, H);
            }
        }
        __syncthreads();
        if constexpr (kBig) {
            if (tid < E) s_run[tid] += chunk_rows;
        } else {
            for (int ee = tid; ee < E; ee += NT) {
                int c = 0;
                for (int w = 0; w < W; ++w) c += __popc(s_bm[ee * W + w]);
                s_run[ee] += c;
            }
        }
        __syncthreads();
    }
}

}  // namespace moe
