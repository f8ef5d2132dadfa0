// k_stream.hip — block-scaled FP4 expert GEMMs on gfx950 matrix cores:
// gate_up (+ SwiGLU + MXFP8 requant) and down, for MXFP4 and NVFP4 experts.
//
// Pages: SGLang-NVIDIA-Mega README, DeepSeek-V4.1 slot table, row "Routed
// experts (moe)" (a pair of block-scaled GEMMs over 8-row tiles; an expert
// with more than 8 rows takes several tiles); README Qwen3.5 slot table, row
// "mkm" (FC1, SwiGLU, requant, FC2); sgl-nvidia-mega PR #24, "Modifications /
// Target spec" (NVFP4 routed experts); SGLang Spark GB10 Optimizations,
// section 1 (NVFP4 K-groups of 16 with FP8 scale rows) and section 4 (a
// sparse FP4 GEMV for MoE decode).
//
// Work decomposition (weight streaming, HBM-bound).  An item is (active
// expert, block of weight rows, K range); activations arrive in bucket order,
// so an expert's rows are contiguous.  After one memory round trip (slot ->
// expert and bucket range) every wave streams its weight rows AND the
// activation rows of its pass through one register ring D steps deep: per
// 128-K step a lane loads its 16 weight bytes, their scales, its 32
// activation bytes and their scale.  No LDS stage, no barrier and no other
// dependent load sits between the expert lookup and the K loop (under load a
// dependent load waits behind every request already queued on the CU, so each
// one costs several microseconds).  The activation bytes of an expert are
// read by all of its workgroups and come from the L2.
//   gate_up over the whole K fuses SwiGLU and the MXFP8 requant; a gate_up
//   split over K (used only when too few items would fill the GPU) writes
//   fp32 partials that a second launch adds in split order; down writes fp32
//   per (row, slot).  Every expert weight byte is read once per call for up
//   to 32 rows per expert; more rows take more passes.
// Loads of rows past the pass, and ring refills past the K range, go through
// a buffer resource at an offset past its record count: they return zeros
// without touching memory, so the loop has no branches (a branch between an
// MFMA and the read of its accumulator is also what the compiler does not
// always pad correctly on this target).
//
// Operand layouts (checked on the hardware):
//   v_mfma_scale_f32_16x16x128_f8f6f4, FP4 operand: lane (row i, group g)
//     holds K [32g, 32g+32) as 16 packed bytes; FP8 operand: lane (col n, g)
//     holds K [16g, 16g+16) in bytes 0-15 and K [64+16g, 64+16g+16) in bytes
//     16-31; the E8M0 scale of (row/col i, K block b) comes from lane 16b+i.
//   v_mfma_f32_16x16x32_f16: lane (i, g) holds K [8g, 8g+8).
//   Output D (16x16): lane l holds D[4(l/16)+r][l%16], r = 0..3.
// Weights are the M side (16 rows per block), activation rows the N side.
// Weights come in the load-order layout of moe_pack_fp4: the 1 KB of A
// operands of a (16-row block, step) is contiguous in lane order, and one
// dword (MX) or two (NV) per lane carry the weight scales of 4 steps (the
// MFMA's op_sel picks an MX scale byte), so each load instruction is dense.
#include "dense_bf16_dev.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "quant_dev.h"
#include "route_dev.h"

#include <algorithm>

namespace moe {

namespace {

constexpr int kFmtMX = MOE_FMT_MXFP4;
constexpr int kFmtNV = MOE_FMT_NVFP4;
constexpr int kFmtNV4 = 16;  // NVFP4 weights with NVFP4 activations (FMT of the templates only)
template <int F>
constexpr bool kNVW = F == kFmtNV || F == kFmtNV4;  // NVFP4 weights
template <int F>
constexpr bool kA4 = F == kFmtNV4;  // NVFP4 activations
constexpr int kThreads = 256;
constexpr int kPassRows = 32;           // activation rows per pass (two 16-row N-blocks)
static_assert(kPassRows % kYGroupRows == 0, "a pass holds whole grouped-y groups");

#ifndef MOE_STREAM_TARGET_ITEMS
#define MOE_STREAM_TARGET_ITEMS 256  // gate_up splits K until about this many items
#endif
#ifndef MOE_RING_LOADS
#define MOE_RING_LOADS 32  // 16-byte loads per lane the register ring may hold
#endif
#ifndef MOE_ROWS_TARGET_WGS
#define MOE_ROWS_TARGET_WGS 512  // down by rows: workgroups to spread an expert set over
#endif
#ifndef MOE_ROWS_MAX_KB
#define MOE_ROWS_MAX_KB 32  // down by rows: most weight KB per wave
#endif
#ifndef MOE_MIN_BLOCKS
#define MOE_MIN_BLOCKS 2  // workgroups per CU the register budget must allow
#endif
#ifndef MOE_MX_DQ
#define MOE_MX_DQ 2  // MXFP4 gate_up with the activation tile in LDS: weight ring depth in quads
#endif
#ifndef MOE_MX_DOWN_DQ
#define MOE_MX_DOWN_DQ 1  // MXFP4 down along K with the h tile in LDS: weight ring depth in quads (four blocks: one)
#endif
#ifndef MOE_NV_DQ
#define MOE_NV_DQ 2  // NVFP4 gate_up: weight ring depth in quads
#endif
#ifndef MOE_NV_MINB
#define MOE_NV_MINB MOE_MIN_BLOCKS  // NVFP4 gate_up: workgroups per CU the register budget must allow
#endif
#ifndef MOE_WEIGHT_AUX
#define MOE_WEIGHT_AUX 2  // cache policy of the weight loads: non-temporal (streamed once)
#endif

struct StreamJob {
    const uint8_t* w;       // packed E2M1, [E][N][K/2]
    const uint8_t* sc;      // MX: E8M0 [E][N][K/32]; NV: E4M3 [E][N][K/16]
    const float* gscale;    // NV: per-expert fp32 global
    int N, K;               // weight rows per expert, reduction length
    int dense;              // one expert over all M rows
    const int32_t* bucket;
    const int32_t* active;
    const int32_t* active_offsets;  // bucket range of each slot
    int M;
    const uint8_t* a_q;     // activation codes [rows][K] (bucket order; token order when dense)
    const uint8_t* a_s;     // activation scales [rows][K/32]
    uint32_t a_rows;        // rows of a_q / a_s (record counts)
    int span;               // K per split (multiple of 128)
    int splits;
    int nblk;               // row blocks per expert
    int out_rows;           // rows of the partial buffer (gate_up split)
    const int32_t* ids;     // routed, M*k <= kThreads pairs: slots resolve from the top-k ids
    int k;                  // top-k (pair id = row * k + slot)
    int a_tok;              // activations in token order: pair p reads row p / k
    const int32_t* count;   // with the active list: the number of active slots (later entries are stale)
    // gate_up resolving from the ids: record the resolved slots here for the
    // down launch (active experts, bucket ranges, count, bucket), or nullptr
    int32_t *r_act, *r_off, *r_na, *r_bkt;
    int2* r_yrec;           // and each pair's grouped-y row (ygroup_rec), or nullptr
    int ygrp;               // down: write y grouped (ygroup_rec) instead of [out_rows][N]
    float limit;            // gate_up: clamped SwiGLU limit (0: unclamped)
    // NVFP4 activations: their global (ag, or age[e] per expert) and the
    // global of the h a gate_up writes (hg, or hge[e])
    float ag, hg;
    const float *age, *hge;
};

__device__ __forceinline__ float act_global(const StreamJob& J, int e) { return J.age ? J.age[e] : J.ag; }
__device__ __forceinline__ float out_global(const StreamJob& J, int e) { return J.hge ? J.hge[e] : J.hg; }

struct Tokens {
    int e, base, n;
    int na;  // active experts (resolve_ids)
};

// Slot -> (expert, bucket range).  The three loads are independent; unused
// slots have no rows.  A dense job's slots are its passes of kPassRows rows
// (so many rows spread over workgroups instead of looping in each).
__device__ __forceinline__ bool resolve(const StreamJob& J, int slot, Tokens& t) {
    if (J.dense) {
        t.e = 0;
        t.base = slot * kPassRows;
        t.n = min(kPassRows, J.M - t.base);
        return t.n > 0;
    }
    const int b0 = J.active_offsets[slot], b1 = J.active_offsets[slot + 1];
    const int e = J.active[slot];
    if (J.count && slot >= *J.count) return false;
    if (b1 <= b0) return false;
    t.e = e;
    t.base = b0;
    t.n = b1 - b0;
    return true;
}

// Item -> (slot, column block) of a dense job, whose slots are passes over
// the same weights: the passes of one column block take consecutive items of
// one XCD (a launch's workgroups go to the eight XCDs in turn), so they run
// together there and the later ones find the weights in that XCD's L2.
// Routed jobs (and a column-block count that is not a multiple of 8) keep
// slot-major items.
__device__ __forceinline__ void item_of(const StreamJob& J, int bid, int nblk, int& slot, int& blk) {
    if (J.dense && nblk % 8 == 0) {
        const int passes = (J.M + kPassRows - 1) / kPassRows;
        const int q = bid >> 3;
        slot = q % passes;
        blk = (q / passes) * 8 + (bid & 7);
    } else {
        slot = bid / nblk;
        blk = bid % nblk;
    }
}

// Slot -> (expert, bucket range) from the top-k ids, for P = M*k <= kIdsPairs
// pairs (two per thread: pairs tid and tid + kThreads): the slot-th chosen
// expert in ascending id order, its bucket base (the pairs with a smaller
// expert) and its pairs in ascending order (list, LDS; tok[t] = list[t] / k),
// the order the route step writes.  One bitmap of the chosen experts in LDS,
// a scan of its word counts in one wave, and per wave one ballot per pair set
// for the pairs below and at the expert.  Every thread of the workgroup calls
// it (it has barriers); the result is uniform.
static_assert(kIdsPairs == 2 * kThreads, "two pairs per thread resolve a slot");
__device__ __forceinline__ bool resolve_ids(const StreamJob& J, int slot, Tokens& t, int* list, int* tok) {
    __shared__ uint32_t s_bm[kMaxE / 32];
    __shared__ int s_cnt[kThreads / 64][3];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int P = J.M * J.k;
    const int id0 = tid < P ? J.ids[tid] : -1;
    const int id1 = tid + kThreads < P ? J.ids[tid + kThreads] : -1;
    if (tid < kMaxE / 32) s_bm[tid] = 0u;
    __syncthreads();
    if (id0 >= 0) atomicOr(&s_bm[id0 >> 5], 1u << (id0 & 31));
    if (id1 >= 0) atomicOr(&s_bm[id1 >> 5], 1u << (id1 & 31));
    __syncthreads();
    const uint32_t word = lane < kMaxE / 32 ? s_bm[lane] : 0u;
    int incl = __popc(word);  // inclusive count of chosen experts up to this word
#pragma unroll
    for (int off = 1; off < kMaxE / 32; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, kMaxE / 32 - 1, 64));
    if (slot >= total) return false;
    const uint64_t over = __ballot(lane < kMaxE / 32 && incl > slot);
    const int w = __ffsll((unsigned long long)over) - 1;  // word holding the expert
    const int before = __shfl(incl - __popc(word), w, 64);
    uint32_t bits = (uint32_t)__shfl((int)word, w, 64);
    for (int r = slot - before; r > 0; --r) bits &= bits - 1u;
    const int e = 32 * w + __ffs(bits) - 1;
    const uint64_t lt0 = __ballot(id0 >= 0 && id0 < e), eq0 = __ballot(id0 == e);
    const uint64_t lt1 = __ballot(id1 >= 0 && id1 < e), eq1 = __ballot(id1 == e);
    if (lane == 0) {
        s_cnt[wave][0] = __popcll(lt0) + __popcll(lt1);
        s_cnt[wave][1] = __popcll(eq0);
        s_cnt[wave][2] = __popcll(eq1);
    }
    __syncthreads();
    int base = 0, n0 = 0, n1 = 0, pre0 = 0, pre1 = 0;
#pragma unroll
    for (int w2 = 0; w2 < kThreads / 64; ++w2) {
        base += s_cnt[w2][0];
        pre0 += w2 < wave ? s_cnt[w2][1] : 0;
        pre1 += w2 < wave ? s_cnt[w2][2] : 0;
        n0 += s_cnt[w2][1];
        n1 += s_cnt[w2][2];
    }
    const uint64_t below = (1ull << lane) - 1ull;
    if (id0 == e) {
        const int pos = pre0 + __popcll(eq0 & below);
        list[pos] = tid;
        tok[pos] = tid / J.k;
    }
    if (id1 == e) {  // pairs tid + kThreads follow all of the first set
        const int pos = n0 + pre1 + __popcll(eq1 & below);
        list[pos] = tid + kThreads;
        tok[pos] = (tid + kThreads) / J.k;
    }
    __syncthreads();
    // uniform, but computed through lane exchanges: say so, or every buffer
    // load through the expert's resource becomes a readfirstlane loop
    t.e = __builtin_amdgcn_readfirstlane(e);
    t.base = __builtin_amdgcn_readfirstlane(base);
    t.n = __builtin_amdgcn_readfirstlane(n0 + n1);
    t.na = total;
    return true;
}

__device__ __forceinline__ bool resolve_item(const StreamJob& J, int slot, Tokens& t, int* list, int* tok) {
    return (J.ids && !J.dense) ? resolve_ids(J, slot, t, list, tok) : resolve(J, slot, t);
}

// ---- NVFP4 helpers ----------------------------------------------------------

// The two E4M3 block scales of one step (bytes 2h, 2h+1 of the dword) ->
// exponent carriers sv0, sv1 for the scaled E2M1 conversion and an f16 pair of
// mantissa factors carrying the scales' signs.  The conversion uses only the
// exponent field of its fp32 scale (its sign and mantissa are ignored, and an
// all-ones exponent, i.e. a NaN scale, makes every output NaN; checked on the
// hardware), so value = conv(e2m1, sv) * m is exact: the E4M3 scale is exact
// in f16, its mantissa field with exponent 0 and the sign kept is m.
template <int H>
__device__ __forceinline__ void nv_scales2(uint32_t dw, float& sv0, float& sv1, v2h& m) {
    sv0 = __builtin_amdgcn_cvt_f32_fp8((int)dw, 2 * H);
    sv1 = __builtin_amdgcn_cvt_f32_fp8((int)dw, 2 * H + 1);
    const v2h sf = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dw, 1.0f, H != 0);
    m = __builtin_bit_cast(v2h, (__builtin_bit_cast(uint32_t, sf) & 0x83FF83FFu) | 0x3C003C00u);
}

// 8 packed E2M1 (one dword) -> 8 f16 = e2m1 * 2^floor(log2 sv) * m (exact).
__device__ __forceinline__ v8h nv_dequant8(uint32_t w, float sv, _Float16 m) {
    const v2h mm = {m, m};
    v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 0) * mm;
    v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 1) * mm;
    v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 2) * mm;
    v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sv, 3) * mm;
    return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 E4M3 activation codes (two dwords) -> 8 f16 scaled by 2^floor(log2 sf).
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t d0, uint32_t d1, float sf) {
    const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, sf, false);
    const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, sf, true);
    const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, sf, false);
    const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, sf, true);
    return v8h{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Per-row factor that turns an NVFP4 accumulator into the product value:
// 2^(smax - 127) (activation offset) * global.
__device__ __forceinline__ float nv_row_factor(int smax, float gs) { return ldexpf(gs, smax - 127); }

// NVFP4 activations enter the f16 MFMA exactly: E2M1 * E4M3 has at most six
// significant bits and lies in [2^-10, 2688].  The lane's 32 codes of a step
// (16 bytes, K [32g, +32)) and the dword holding its two scale bytes (bytes
// 2(g & 1), +1) -> the four B operands (the order nv_dequant8 gives weights).
__device__ __forceinline__ void act4_to_f16(const v4i& b, uint32_t sdw, int g, v8h (&B)[4]) {
    float sv0, sv1;
    v2h m;
    nv_scales2<0>(sdw >> (16 * (g & 1)), sv0, sv1, m);
    B[0] = nv_dequant8((uint32_t)b.x, sv0, m[0]);
    B[1] = nv_dequant8((uint32_t)b.y, sv0, m[0]);
    B[2] = nv_dequant8((uint32_t)b.z, sv1, m[1]);
    B[3] = nv_dequant8((uint32_t)b.w, sv1, m[1]);
}

// ---- coordinates and the ring -------------------------------------------------

// Per-lane coordinates: MB blocks of 16 weight rows (packed layout), NB blocks
// of 16 activation rows.
template <int FMT, int MB, int NB>
struct Coord {
    __amdgpu_buffer_rsrc_t rw, rs, ra, ras;
    uint32_t vw[MB];   // the lane's 16 bytes of step 0 of its weight block
    uint32_t vs[MB];   // the lane's scale entry of quad 0 of its weight block
    uint32_t va[NB];   // activation bytes of the lane's row (kOOB past the pass)
    uint32_t vas[NB];  // activation scale dword of step 0 of the lane's row (kOOB past the pass)
};

// wblk: first row of each weight block (a multiple of 16).  src: the a_q row
// of each pass row (LDS), or nullptr for rows arow0, arow0 + 1, ...
template <int FMT, int MB, int NB>
__device__ __forceinline__ Coord<FMT, MB, NB> make_coord(const StreamJob& J, int e, const int (&wblk)[MB],
                                                          int arow0, int npass, const int* src) {
    const int lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    const int K = J.K, S = K / 128, Q = (S + 3) / 4;
    constexpr int SQ = FMT == kFmtMX ? 256 : 512;  // scale bytes per (block, quad)
    const uint32_t wbytes = (uint32_t)J.N * (K / 2);
    const uint32_t sbytes = (uint32_t)(J.N / 16) * Q * SQ;
    Coord<FMT, MB, NB> c;
    c.rw = make_rsrc(J.w + (size_t)e * wbytes, wbytes);
    c.rs = make_rsrc(J.sc + (size_t)e * sbytes, sbytes);
    // activation row bytes: MXFP8 K codes + K/32 scales; NVFP4 K/2 + K/16
    const int AQ = kA4<FMT> ? K / 2 : K, AS = kA4<FMT> ? K / 16 : K / 32;
    if (src) {  // gathered rows: the resources cover all of a_q
        c.ra = make_rsrc(J.a_q, J.a_rows * (uint32_t)AQ);
        c.ras = make_rsrc(J.a_s, J.a_rows * (uint32_t)AS);
    } else {  // the pass's rows only (offsets stay small)
        const uint32_t prow = (uint32_t)min(kPassRows, (int)J.a_rows - arow0);
        c.ra = make_rsrc(J.a_q + (size_t)arow0 * AQ, prow * (uint32_t)AQ);
        c.ras = make_rsrc(J.a_s + (size_t)arow0 * AS, prow * (uint32_t)AS);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const uint32_t rb = (uint32_t)wblk[mb] / 16;
        c.vw[mb] = rb * S * 1024 + 16 * lane;
        c.vs[mb] = rb * Q * SQ + (SQ / 64) * lane;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int t = 16 * j + i;
        const bool ok = t < npass;
        const uint32_t r = ok ? (src ? (uint32_t)src[t] : (uint32_t)t) : 0u;
        // MX: bytes [16g, +16) and [64 + 16g, +16) of the step; NV: [32g, +32);
        // NVFP4 activations: [16g, +16) of the step's 64, and the scale dword
        // holding the lane's two scale bytes (2g, 2g + 1 of the step's 8)
        if constexpr (kA4<FMT>) {
            c.va[j] = ok ? r * (uint32_t)(K / 2) + 16 * g : kOOB;
            c.vas[j] = ok ? r * (uint32_t)(K / 16) + 4 * (g >> 1) : kOOB;
        } else {
            c.va[j] = ok ? r * K + (FMT == kFmtMX ? 16 : 32) * g : kOOB;
            c.vas[j] = ok ? r * (K / 32) : kOOB;
        }
    }
    return c;
}

// A ring slot holds one quad: QS K steps (4, or fewer when the whole K is
// shorter than a quad) and the weight scales of the quad.
template <int MB, int NB, int DQ, int QS>
struct Ring {
    v4i a[DQ][QS][MB];
    uint32_t as[DQ][MB][2];
    v4i b[DQ][QS][NB][2];
    uint32_t bs[DQ][QS][NB];
};

// Loads step u of quad q (absolute) into slot v; steps at or past s_end load zeros.
template <int FMT, int MB, int NB, int DQ, int QS>
__device__ __forceinline__ void ring_load_step(Ring<MB, NB, DQ, QS>& R, int v, int u, const Coord<FMT, MB, NB>& c,
                                               int q, int s_end) {
    const int st = 4 * q + u;
    const bool ok = st < s_end;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        R.a[v][u][mb] = __builtin_amdgcn_raw_buffer_load_b128(c.rw, ok ? c.vw[mb] : kOOB, 1024 * st, MOE_WEIGHT_AUX);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const uint32_t va = ok ? c.va[j] : kOOB;
        if constexpr (kA4<FMT>) {
            R.b[v][u][j][0] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, va, 64 * st, 0);
            R.bs[v][u][j] = __builtin_amdgcn_raw_buffer_load_b32(c.ras, ok ? c.vas[j] : kOOB, 8 * st, 0);
        } else {
            R.b[v][u][j][0] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, va, 128 * st, 0);
            R.b[v][u][j][1] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, va + (FMT == kFmtMX ? 64 : 16), 128 * st, 0);
            R.bs[v][u][j] = __builtin_amdgcn_raw_buffer_load_b32(c.ras, ok ? c.vas[j] : kOOB, 4 * st, 0);
        }
    }
}

// Loads the weight scales of quad q (absolute) into slot v.
template <int FMT, int MB, int NB, int DQ, int QS>
__device__ __forceinline__ void ring_load_scales(Ring<MB, NB, DQ, QS>& R, int v, const Coord<FMT, MB, NB>& c, int q,
                                                 int s_end) {
    const bool okq = 4 * q < s_end;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        if constexpr (FMT == kFmtMX) {
            R.as[v][mb][0] = __builtin_amdgcn_raw_buffer_load_b32(c.rs, okq ? c.vs[mb] : kOOB, 256 * q, 0);
        } else {
            const auto sv = __builtin_amdgcn_raw_buffer_load_b64(c.rs, okq ? c.vs[mb] : kOOB, 512 * q, 0);
            R.as[v][mb][0] = sv[0];
            R.as[v][mb][1] = sv[1];
        }
    }
}

// One K step (U of its quad) from operands in registers: a[mb] the weight
// bytes of block mb, as[mb] its quad scale entry, b[j] the activation bytes of
// N-block j, bs[j] their scale dword.
template <int FMT, int MB, int NB, int U>
__device__ __forceinline__ void mfma_step(const v4i (&a_)[MB], const uint32_t (&as)[MB][2], const v4i (&b)[NB][2],
                                          const uint32_t (&bs)[NB], const int (&sfo)[NB], v4f (&acc)[MB][2]) {
    const int g = (threadIdx.x & 63) >> 4;
    if constexpr (FMT == kFmtMX) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const v4i a = a_[mb];
            const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const v4i b0 = b[j][0], b1 = b[j][1];
                const v8i B = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                // A scale: byte U of the quad's dword; B scale: byte g of the step's dword
                acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[mb][j], 4, 0, U, (int)as[mb][0],
                                                                              0, (int)(bs[j] >> (8 * g)));
            }
        }
    } else {
        v8h B[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (kA4<FMT>) {
                act4_to_f16(b[j][0], bs[j], g, B[j]);
            } else {
                const v4i b0 = b[j][0], b1 = b[j][1];
                const int sb = (int)((bs[j] >> (8 * g)) & 0xffu);
                const float sf = exp2i(max(sb + sfo[j], -126));
                B[j][0] = fp8x8_to_f16((uint32_t)b0.x, (uint32_t)b0.y, sf);
                B[j][1] = fp8x8_to_f16((uint32_t)b0.z, (uint32_t)b0.w, sf);
                B[j][2] = fp8x8_to_f16((uint32_t)b1.x, (uint32_t)b1.y, sf);
                B[j][3] = fp8x8_to_f16((uint32_t)b1.z, (uint32_t)b1.w, sf);
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const v4i a = a_[mb];
            float sv0, sv1;
            v2h m;
            nv_scales2<U & 1>(as[mb][U >> 1], sv0, sv1, m);
            const v8h A0 = nv_dequant8((uint32_t)a.x, sv0, m[0]);
            const v8h A1 = nv_dequant8((uint32_t)a.y, sv0, m[0]);
            const v8h A2 = nv_dequant8((uint32_t)a.z, sv1, m[1]);
            const v8h A3 = nv_dequant8((uint32_t)a.w, sv1, m[1]);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B[j][0], acc[mb][j], 0, 0, 0);
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B[j][1], acc[mb][j], 0, 0, 0);
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, B[j][2], acc[mb][j], 0, 0, 0);
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, B[j][3], acc[mb][j], 0, 0, 0);
            }
        }
    }
}

// Step u of the quad in slot v.
template <int FMT, int MB, int NB, int DQ, int QS, int U>
__device__ __forceinline__ void step_mfma(const Ring<MB, NB, DQ, QS>& R, int v, const int (&sfo)[NB],
                                          v4f (&acc)[MB][2]) {
    mfma_step<FMT, MB, NB, U>(R.a[v][U], R.as[v], R.b[v][U], R.bs[v][U], sfo, acc);
}

// NVFP4: largest E8M0 code of the lane's activation row(s) over K steps
// [s0, s0 + nst) (activations enter the f16 MFMA as E4M3 * 2^(s - smax),
// inside f16 range); 0 for rows past the pass.  Two phases: the loads are
// issued before the operand ring is filled and reduced after it, so their
// round trip overlaps the ring's instead of preceding it.  The four lanes of a
// row (g = 0..3) load 16 bytes each per round: dwords 4(g + 4u) .. +3 of the
// range (dword d = the scale bytes of step s0 + d), u < kSmaxU; a range longer
// than 16 * kSmaxU dwords finishes with a loop.
constexpr int kSmaxU = 4;

template <int NB>
struct SmaxRaw {
    v4i v[NB][kSmaxU];
};

template <int FMT, int MB, int NB>
__device__ __forceinline__ void row_smax_issue(const Coord<FMT, MB, NB>& c, int s0, int nst, SmaxRaw<NB>& R) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const bool ok = c.vas[j] != kOOB;
#pragma unroll
        for (int u = 0; u < kSmaxU; ++u) {
            const int d = 4 * (g + 4 * u);
            R.v[j][u] = __builtin_amdgcn_raw_buffer_load_b128(
                c.ras, ok && d < nst ? c.vas[j] + 4 * (s0 + d) : kOOB, 0, 0);
        }
    }
}

__device__ __forceinline__ uint32_t max_byte(uint32_t v) {
    return max(max(v & 0xffu, (v >> 8) & 0xffu), max((v >> 16) & 0xffu, v >> 24));
}

template <int FMT, int MB, int NB>
__device__ __forceinline__ void row_smax_finish(const Coord<FMT, MB, NB>& c, int s0, int nst, const SmaxRaw<NB>& R,
                                                int (&smax)[NB]) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        uint32_t mx = 0;
#pragma unroll
        for (int u = 0; u < kSmaxU; ++u) {
            const int d = 4 * (g + 4 * u);
            const v4i v = R.v[j][u];
            // dwords past the range are ignored (a range may end inside the load)
            mx = max(mx, d + 0 < nst ? max_byte((uint32_t)v.x) : 0u);
            mx = max(mx, d + 1 < nst ? max_byte((uint32_t)v.y) : 0u);
            mx = max(mx, d + 2 < nst ? max_byte((uint32_t)v.z) : 0u);
            mx = max(mx, d + 3 < nst ? max_byte((uint32_t)v.w) : 0u);
        }
        const bool ok = c.vas[j] != kOOB;
        for (int d = 16 * kSmaxU + g; d < nst; d += 4) {
            const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(c.ras, ok ? c.vas[j] + 4 * (s0 + d) : kOOB, 0, 0);
            mx = max(mx, max_byte(v));
        }
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
        smax[j] = (int)mx;
    }
}

// Steps U..QS-1 of the quad in slot v, each followed by its refill with quad
// qn; the quad's scales are refilled after its last step, before that step's
// refill.
template <int FMT, int MB, int NB, int DQ, int QS, int U>
__device__ __forceinline__ void quad_steps(Ring<MB, NB, DQ, QS>& R, int v, const Coord<FMT, MB, NB>& c, int qn,
                                           int s_end, const int (&sfo)[NB], v4f (&acc)[MB][2]) {
    if constexpr (U < QS) {
        // keep each step's instructions in place: hoisting the use of a later
        // slot would wait for that slot's loads and drain the ring
        __builtin_amdgcn_sched_barrier(0);
        step_mfma<FMT, MB, NB, DQ, QS, U>(R, v, sfo, acc);
        if constexpr (U == QS - 1) ring_load_scales<FMT, MB, NB, DQ, QS>(R, v, c, qn, s_end);
        ring_load_step<FMT, MB, NB, DQ, QS>(R, v, U, c, qn, s_end);
        quad_steps<FMT, MB, NB, DQ, QS, U + 1>(R, v, c, qn, s_end, sfo, acc);
    }
}

// All of one pass: K steps [s0, s0 + nst) (s0 a multiple of 4) of MB weight
// blocks against NB blocks of activation rows arow0 + [0, npass).  The ring
// holds DQ quads; each step's slot is refilled right after its MFMAs, so
// DQ*QS - 1 steps stay in flight.  Steps past the range load zeros for both
// operands.
template <int FMT, int MB, int NB, int DQ, int QS>
__device__ __forceinline__ void stream_pass(const StreamJob& J, int e, const int (&wblk)[MB], int arow0, int npass,
                                            const int* src, int s0, int nst, int (&smax)[NB], v4f (&acc)[MB][2]) {
    const Coord<FMT, MB, NB> c = make_coord<FMT, MB, NB>(J, e, wblk, arow0, npass, src);
    SmaxRaw<NB> SR;
    if constexpr (FMT == kFmtNV) row_smax_issue<FMT, MB, NB>(c, s0, nst, SR);
    const int q0 = s0 / 4, nq = (nst + 3) / 4, s_end = s0 + nst;
    Ring<MB, NB, DQ, QS> R;
    // Fill the ring in the order the loop refills it (a quad's scales with its
    // last step).  The wait counts at the loop head are merged over the entry
    // and the back edge; an entry order with the scales issued last would
    // make the first use of a quad's scales wait for every load in flight.
    static_assert(QS == 4, "the ring streams whole quads");
#pragma unroll
    for (int v = 0; v < DQ; ++v) {
#pragma unroll
        for (int u = 0; u < QS; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            if (u == QS - 1) ring_load_scales<FMT, MB, NB, DQ, QS>(R, v, c, q0 + v, s_end);
            ring_load_step<FMT, MB, NB, DQ, QS>(R, v, u, c, q0 + v, s_end);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    int sfo[NB];
    if constexpr (FMT == kFmtNV) {
        row_smax_finish<FMT, MB, NB>(c, s0, nst, SR, smax);
#pragma unroll
        for (int j = 0; j < NB; ++j) sfo[j] = -smax[j];
    } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            sfo[j] = 0;
            smax[j] = 0;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int l0 = 0; l0 < nq; l0 += DQ) {
#pragma unroll
        for (int v = 0; v < DQ; ++v)
            quad_steps<FMT, MB, NB, DQ, QS, 0>(R, v, c, q0 + l0 + v + DQ, s_end, sfo, acc);
    }
}

// ---- NVFP4: streaming with the activation tile of a quad in LDS --------------
// The four waves of a workgroup use the same activation rows.  The workgroup
// loads the tile of a quad (16*NB rows x 512 K) once, a share per thread,
// converts it to the f16 operand form (E4M3 * 2^(s - smax), smax the row's
// largest scale code over the item's K range) and stores it into one of two
// LDS buffers; the waves read ready operands from there, and the register
// ring holds weights only.  One barrier per quad: tile q+1 is written while
// tile q is read, the barrier publishes it.
constexpr int kTileRowH = 1040;  // bytes per row: 512 f16 + 16 (staggers banks)
// one buffer of a pass of NB N-blocks
template <int NB>
constexpr int tile_bytes_h() {
    return 16 * NB * kTileRowH;
}

template <int NB>
struct ActShare {
    v4i c[2 * NB];       // code chunks of the thread (16 codes each)
    uint32_t s[2 * NB];  // the E8M0 code of each chunk's 32-block
};

// The thread's share of a tile: byte offsets (in a_q, a_s) of its code chunks
// and of their scale bytes at quad 0; kOOB for rows past the pass.  Chunk k of
// thread t is row (t + 256k) / 32, codes [16 ch, +16) of the quad, ch =
// (t + 256k) % 32.  src as in make_coord.
template <int NB>
struct TileOffs {
    uint32_t c[2 * NB];
    uint32_t s[2 * NB];
};

// A4 (NVFP4 activations): a chunk is 8 code bytes (16 values) and its one
// E4M3 scale byte.
template <int NB, bool A4>
__device__ __forceinline__ TileOffs<NB> tile_offsets(int K, int npass, const int* src) {
    const int t = threadIdx.x;
    TileOffs<NB> o;
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
        const int li = t + kThreads * k, row = li >> 5, ch = li & 31;
        const uint32_t r = row < npass ? (src ? (uint32_t)src[row] : (uint32_t)row) : 0u;
        if constexpr (A4) {
            o.c[k] = row < npass ? r * (uint32_t)(K / 2) + 8 * ch : kOOB;
            o.s[k] = row < npass ? r * (uint32_t)(K / 16) + ch : kOOB;
        } else {
            o.c[k] = row < npass ? r * (uint32_t)K + 16 * ch : kOOB;
            o.s[k] = row < npass ? r * (uint32_t)(K / 32) + (ch >> 1) : kOOB;
        }
    }
    return o;
}

// Requests the thread's share of tile q (absolute quad).  Rows past the pass
// and steps at or past s_end read zeros.
template <int NB, bool A4, int CF>
__device__ __forceinline__ void tile_load(ActShare<NB>& P, const Coord<CF, 1, NB>& c, const TileOffs<NB>& o,
                                          int q, int s_end) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
        const int ch = (t + kThreads * k) & 31;
        const bool ok = o.c[k] != kOOB && 4 * q + (ch >> 3) < s_end;
        if constexpr (A4) {
            const auto cv = __builtin_amdgcn_raw_buffer_load_b64(c.ra, ok ? o.c[k] + 256 * q : kOOB, 0, 0);
            P.c[k] = v4i{(int)cv[0], (int)cv[1], 0, 0};
            P.s[k] = __builtin_amdgcn_raw_buffer_load_b8(c.ras, ok ? o.s[k] + 32 * q : kOOB, 0, 0);
        } else {
            P.c[k] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, ok ? o.c[k] + 512 * q : kOOB, 0, 0);
            P.s[k] = __builtin_amdgcn_raw_buffer_load_b8(c.ras, ok ? o.s[k] + 16 * q : kOOB, 0, 0);
        }
    }
}

// Converts the thread's share of a tile to f16 and writes it into an LDS
// buffer.  rsmax: the pass rows' smax (LDS).  Codes past the range are zero,
// and so are their f16 values.  A wave whose two rows of a round are both
// past the pass skips that round: those LDS rows keep stale values, which
// reach only the MFMA output columns of rows past the pass (each output
// column depends on its own B column only), and those are never stored.
template <int NB, bool A4>
__device__ __forceinline__ void tile_store(const ActShare<NB>& P, uint8_t* buf, const int* rsmax, int npass) {
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
        if (8 * k + 2 * wave >= npass) continue;  // uniform: rows 8k + 2w, +1 of the wave
        const int li = t + kThreads * k, row = li >> 5, ch = li & 31;
        v8h h0, h1;
        if constexpr (A4) {
            // exact: E2M1 * E4M3 (the scale's exponent carrier times its mantissa factor)
            float sv0, sv1;
            v2h m;
            nv_scales2<0>(P.s[k] & 0xffu, sv0, sv1, m);
            h0 = nv_dequant8((uint32_t)P.c[k].x, sv0, m[0]);
            h1 = nv_dequant8((uint32_t)P.c[k].y, sv0, m[0]);
        } else {
            const int sm = row < npass ? rsmax[row] : 0;
            const float sf = exp2i(max((int)(P.s[k] & 0xffu) - sm, -126));
            h0 = fp8x8_to_f16((uint32_t)P.c[k].x, (uint32_t)P.c[k].y, sf);
            h1 = fp8x8_to_f16((uint32_t)P.c[k].z, (uint32_t)P.c[k].w, sf);
        }
        uint8_t* p = buf + row * kTileRowH + 32 * ch;
        *reinterpret_cast<v8h*>(p) = h0;
        *reinterpret_cast<v8h*>(p + 16) = h1;
    }
}

// The lane's B operands of step u of the tile in buf: row 16j + i, K
// [128u + 32g + 8c, +8) for MFMA c (the order nv_dequant8 gives the weights).
template <int NB>
__device__ __forceinline__ void tile_read(const uint8_t* buf, int u, v8h (&B)[NB][4]) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const uint8_t* p = buf + (16 * j + i) * kTileRowH + 256 * u + 64 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) B[j][c] = *reinterpret_cast<const v8h*>(p + 16 * c);
    }
}

// One NVFP4 K step with f16 activation operands given.
template <int MB, int NB, int U>
__device__ __forceinline__ void mfma_step_h(const v4i (&a_)[MB], const uint32_t (&as)[MB][2], const v8h (&B)[NB][4],
                                            v4f (&acc)[MB][2]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const v4i a = a_[mb];
        float sv0, sv1;
        v2h m;
        nv_scales2<U & 1>(as[mb][U >> 1], sv0, sv1, m);
        const v8h A0 = nv_dequant8((uint32_t)a.x, sv0, m[0]);
        const v8h A1 = nv_dequant8((uint32_t)a.y, sv0, m[0]);
        const v8h A2 = nv_dequant8((uint32_t)a.z, sv1, m[1]);
        const v8h A3 = nv_dequant8((uint32_t)a.w, sv1, m[1]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B[j][0], acc[mb][j], 0, 0, 0);
            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B[j][1], acc[mb][j], 0, 0, 0);
            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, B[j][2], acc[mb][j], 0, 0, 0);
            acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, B[j][3], acc[mb][j], 0, 0, 0);
        }
    }
}

// Weight ring: DQ quads of MB blocks.
template <int MB, int DQ>
struct RingW {
    v4i a[DQ][4][MB];
    uint32_t as[DQ][MB][2];
};

template <int MB, int NB, int DQ, int CF>
__device__ __forceinline__ void ringw_load_step(RingW<MB, DQ>& R, int v, int u, const Coord<CF, MB, NB>& c, int q,
                                                int s_end) {
    const int st = 4 * q + u;
    const bool ok = st < s_end;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        R.a[v][u][mb] = __builtin_amdgcn_raw_buffer_load_b128(c.rw, ok ? c.vw[mb] : kOOB, 1024 * st, MOE_WEIGHT_AUX);
}

template <int MB, int NB, int DQ, int CF>
__device__ __forceinline__ void ringw_load_scales(RingW<MB, DQ>& R, int v, const Coord<CF, MB, NB>& c, int q,
                                                  int s_end) {
    const bool okq = 4 * q < s_end;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const auto sv = __builtin_amdgcn_raw_buffer_load_b64(c.rs, okq ? c.vs[mb] : kOOB, 512 * q, 0);
        R.as[v][mb][0] = sv[0];
        R.as[v][mb][1] = sv[1];
    }
}

// The four steps of the quad in slot v, the B operands of step U given and
// those of step U+1 read from the tile meanwhile; each step's weight slot is
// refilled with quad qn right after its MFMAs.
template <int MB, int NB, int DQ, int U, int CF>
__device__ __forceinline__ void quadw_steps(RingW<MB, DQ>& R, int v, const Coord<CF, MB, NB>& c, int qn,
                                            int s_end, const uint8_t* tile, const v8h (&B)[NB][4],
                                            v4f (&acc)[MB][2]) {
    if constexpr (U < 4) {
        __builtin_amdgcn_sched_barrier(0);
        v8h Bn[NB][4];
        if constexpr (U < 3) tile_read<NB>(tile, U + 1, Bn);
        mfma_step_h<MB, NB, U>(R.a[v][U], R.as[v], B, acc);
        if constexpr (U == 3) ringw_load_scales<MB, NB, DQ>(R, v, c, qn, s_end);
        ringw_load_step<MB, NB, DQ>(R, v, U, c, qn, s_end);
        quadw_steps<MB, NB, DQ, U + 1>(R, v, c, qn, s_end, tile, Bn, acc);
    }
}

// An NVFP4 pass as stream_pass, with the activation tiles in LDS (tiles: two
// tile_bytes_h<LB>() buffers, LB the N-blocks the layout is sized for; rsmax:
// 16 * NB ints).  Every thread of the workgroup
// must call it with the same arguments apart from the weight blocks (it has
// barriers).
template <int MB, int NB, int DQ, bool A4, int LB>
__device__ __forceinline__ void stream_pass_lds(const StreamJob& J, int e, const int (&wblk)[MB], int arow0,
                                                int npass, const int* src, int s0, int nst, int (&smax)[NB],
                                                v4f (&acc)[MB][2], uint8_t* tiles, int* rsmax) {
    constexpr int CF = A4 ? kFmtNV4 : kFmtNV;
    const Coord<CF, MB, NB> c = make_coord<CF, MB, NB>(J, e, wblk, arow0, npass, src);
    const TileOffs<NB> to = tile_offsets<NB, A4>(J.K, npass, src);
    Coord<CF, 1, NB> ca;  // the activation resources, for the tile loads
    ca.ra = c.ra;
    ca.ras = c.ras;
    SmaxRaw<NB> SR;
    if constexpr (!A4) row_smax_issue<kFmtNV, MB, NB>(c, s0, nst, SR);
    __builtin_amdgcn_sched_barrier(0);
    const int q0 = s0 / 4, nq = (nst + 3) / 4, s_end = s0 + nst;
    ActShare<NB> P;
    tile_load<NB, A4>(P, ca, to, q0, s_end);
    RingW<MB, DQ> R;
#pragma unroll
    for (int v = 0; v < DQ; ++v) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            if (u == 3) ringw_load_scales<MB, NB, DQ>(R, v, c, q0 + v, s_end);
            ringw_load_step<MB, NB, DQ>(R, v, u, c, q0 + v, s_end);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (A4) {
#pragma unroll
        for (int j = 0; j < NB; ++j) smax[j] = 0;
    } else {
        row_smax_finish<kFmtNV, MB, NB>(c, s0, nst, SR, smax);
        __builtin_amdgcn_sched_barrier(0);
        // every wave holds the rows' smax; wave 0 publishes them for the tile stores
        if (threadIdx.x < 16) {
#pragma unroll
            for (int j = 0; j < NB; ++j) rsmax[16 * j + threadIdx.x] = smax[j];
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    tile_store<NB, A4>(P, tiles + (q0 & 1) * tile_bytes_h<LB>(), rsmax, npass);  // the tile of quad q sits in buffer q & 1
    __syncthreads();
    for (int l0 = 0; l0 < nq; l0 += DQ) {
#pragma unroll
        for (int v = 0; v < DQ; ++v) {
            const int q = q0 + l0 + v;  // the quad of slot v in this round
            const uint8_t* tile = tiles + (q & 1) * tile_bytes_h<LB>();
            v8h B[NB][4];
            tile_read<NB>(tile, 0, B);
            tile_load<NB, A4>(P, ca, to, q + 1, s_end);  // in flight over the quad's steps
            quadw_steps<MB, NB, DQ, 0>(R, v, c, q + DQ, s_end, tile, B, acc);
            // tile q+1 into the other buffer (its reads ended at the last barrier)
            tile_store<NB, A4>(P, tiles + ((q + 1) & 1) * tile_bytes_h<LB>(), rsmax, npass);
            __syncthreads();
        }
    }
}

// ---- MXFP4: streaming with the MXFP8 activation tile of a quad in LDS --------
// With many rows per expert a wave loads as many activation bytes per step as
// weight bytes, and the four waves of a workgroup load the same rows (from the
// cache).  Instead the workgroup loads the tile of a quad once: 16*NB rows x
// 512 E4M3 codes and their 16 E8M0 scale bytes per row, a share per thread,
// into one of two LDS buffers; the waves read their B operands from there and
// the register ring holds weights only.  One barrier per quad, as in the
// NVFP4 path.  Rows are 528 bytes apart (512 codes + 16): the 16 rows a
// wave's lanes read at one step start on 16 different bank groups, and a
// lane's reads of the quad's steps are immediate offsets from one address.
constexpr int kTileRowMX = 528;  // row stride of the codes (512 + 16)
// One buffer of a pass of NB N-blocks: the codes, the rows' scale bytes, and a
// dump area where threads without a scale dword store theirs: every store of
// the tile is unconditional, so the loop body stays one basic block (a branch
// there lets the compiler sink the MFMAs past the barriers).
template <int NB>
constexpr int tile_codes_mx() {
    return 16 * NB * kTileRowMX;
}
template <int NB>
constexpr int tile_scales_mx() {
    return 16 * NB * 16;
}
template <int NB>
constexpr int tile_bytes_mx() {
    return tile_codes_mx<NB>() + tile_scales_mx<NB>() + 4 * kThreads;
}

template <int NB>
struct ActShareMX {
    v4i c[2 * NB];  // code chunks of the thread (16 codes each)
    uint32_t s;     // a scale dword of the thread (threads below 64 * NB)
};

template <int NB>
struct TileOffsMX {
    uint32_t c[2 * NB];  // byte offsets in a_q of the thread's chunks at quad 0 (kOOB past the pass)
    uint32_t s;          // byte offset in a_s of the thread's scale dword at quad 0 (kOOB: none)
};

// Chunk k of thread t is row (t + 256k) / 32, codes [16 ch, +16) of the quad,
// ch = (t + 256k) % 32; thread t < 64 NB loads dword t % 4 of row t / 4's 16
// scale bytes.  src as in make_coord.
template <int NB>
__device__ __forceinline__ TileOffsMX<NB> tile_offsets_mx(int K, int npass, const int* src) {
    const int t = threadIdx.x;
    TileOffsMX<NB> o;
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
        const int li = t + kThreads * k, row = li >> 5, ch = li & 31;
        const uint32_t r = row < npass ? (src ? (uint32_t)src[row] : (uint32_t)row) : 0u;
        o.c[k] = row < npass ? r * (uint32_t)K + 16 * ch : kOOB;
    }
    const int srow = t >> 2;
    const uint32_t rs = srow < npass ? (src ? (uint32_t)src[srow] : (uint32_t)srow) : 0u;
    o.s = (t < 64 * NB && srow < npass) ? rs * (uint32_t)(K / 32) + 4 * (t & 3) : kOOB;
    return o;
}

// Requests the thread's share of tile q (absolute quad); rows past the pass
// and steps at or past s_end read zeros.
template <int NB>
__device__ __forceinline__ void tile_load_mx(ActShareMX<NB>& P, const Coord<kFmtMX, 1, NB>& c,
                                             const TileOffsMX<NB>& o, int q, int s_end) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
        const int ch = (t + kThreads * k) & 31;
        const bool ok = o.c[k] != kOOB && 4 * q + (ch >> 3) < s_end;
        P.c[k] = __builtin_amdgcn_raw_buffer_load_b128(c.ra, ok ? o.c[k] + 512 * q : kOOB, 0, 0);
    }
    // dword t % 4 holds the scales of step 4q + t % 4
    const bool oks = o.s != kOOB && 4 * q + (t & 3) < s_end;
    P.s = __builtin_amdgcn_raw_buffer_load_b32(c.ras, oks ? o.s + 16 * q : kOOB, 0, 0);
}

// LB: the N-blocks the buffer layout is sized for (the kernel's largest pass).
template <int NB, int LB>
__device__ __forceinline__ void tile_store_mx(const ActShareMX<NB>& P, uint8_t* buf) {
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
        const int li = t + kThreads * k, row = li >> 5, ch = li & 31;
        *reinterpret_cast<v4i*>(buf + row * kTileRowMX + 16 * ch) = P.c[k];
    }
    *reinterpret_cast<uint32_t*>(buf + tile_codes_mx<LB>() + (t < 64 * NB ? 4 * t : tile_scales_mx<LB>() + 4 * t)) =
        P.s;
}

// The lane's B operand of step u of the tile in buf for N-block j: row
// 16j + i, codes [128u + 16g, +16) and [128u + 64 + 16g, +16) (the layout of
// the FP8 operand of the scaled MFMA), and the row's scale dword of step u.
template <int NB, int LB>
__device__ __forceinline__ void tile_read_mx(const uint8_t* buf, int u, v8i (&B)[NB], uint32_t (&bs)[NB]) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int row = 16 * j + i;
        const uint8_t* p = buf + row * kTileRowMX + 16 * g;
        const v4i c0 = *reinterpret_cast<const v4i*>(p + 128 * u);
        const v4i c1 = *reinterpret_cast<const v4i*>(p + 128 * u + 64);
        B[j] = v8i{c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        bs[j] = *reinterpret_cast<const uint32_t*>(buf + tile_codes_mx<LB>() + 16 * row + 4 * u);
    }
}

template <int MB, int NB, int DQ>
__device__ __forceinline__ void ringw_load_scales_mx(RingW<MB, DQ>& R, int v, const Coord<kFmtMX, MB, NB>& c, int q,
                                                     int s_end) {
    const bool okq = 4 * q < s_end;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        R.as[v][mb][0] = __builtin_amdgcn_raw_buffer_load_b32(c.rs, okq ? c.vs[mb] : kOOB, 256 * q, 0);
}

// The four steps of the quad in slot v, the B operands of step U given and
// those of step U+1 read from the tile meanwhile; each step's weight slot is
// refilled with quad qn right after its MFMAs.
template <int MB, int NB, int DQ, int LB, int U>
__device__ __forceinline__ void quadw_steps_mx(RingW<MB, DQ>& R, int v, const Coord<kFmtMX, MB, NB>& c, int qn,
                                               int s_end, const uint8_t* tile, const v8i (&B)[NB],
                                               const uint32_t (&bs)[NB], v4f (&acc)[MB][2]) {
    if constexpr (U < 4) {
        __builtin_amdgcn_sched_barrier(0);
        v8i Bn[NB];
        uint32_t bsn[NB];
        if constexpr (U < 3) tile_read_mx<NB, LB>(tile, U + 1, Bn, bsn);
        const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const v4i a = R.a[v][U][mb];
            const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[j], acc[mb][j], 4, 0, U,
                                                                              (int)R.as[v][mb][0], 0,
                                                                              (int)(bs[j] >> (8 * g)));
        }
        if constexpr (U == 3) ringw_load_scales_mx<MB, NB, DQ>(R, v, c, qn, s_end);
        ringw_load_step<MB, NB, DQ>(R, v, U, c, qn, s_end);
        quadw_steps_mx<MB, NB, DQ, LB, U + 1>(R, v, c, qn, s_end, tile, Bn, bsn, acc);
    }
}

// An MXFP4 pass as stream_pass, with the activation tiles in LDS (tiles: two
// tile_bytes_mx<LB>() buffers).  Every thread of the workgroup must call it with the
// same arguments apart from the weight blocks (it has barriers).
template <int MB, int NB, int DQ, int LB>
__device__ __forceinline__ void stream_pass_lds_mx(const StreamJob& J, int e, const int (&wblk)[MB], int arow0,
                                                   int npass, const int* src, int s0, int nst, v4f (&acc)[MB][2],
                                                   uint8_t* tiles) {
    const Coord<kFmtMX, MB, NB> c = make_coord<kFmtMX, MB, NB>(J, e, wblk, arow0, npass, src);
    const TileOffsMX<NB> to = tile_offsets_mx<NB>(J.K, npass, src);
    Coord<kFmtMX, 1, NB> ca;  // the activation resources, for the tile loads
    ca.ra = c.ra;
    ca.ras = c.ras;
    const int q0 = s0 / 4, nq = (nst + 3) / 4, s_end = s0 + nst;
    ActShareMX<NB> P;
    tile_load_mx<NB>(P, ca, to, q0, s_end);
    RingW<MB, DQ> R;
#pragma unroll
    for (int v = 0; v < DQ; ++v) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            if (u == 3) ringw_load_scales_mx<MB, NB, DQ>(R, v, c, q0 + v, s_end);
            ringw_load_step<MB, NB, DQ>(R, v, u, c, q0 + v, s_end);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // the tile of quad q sits in buffer q & 1
    __syncthreads();  // the previous pass's reads of the LDS are done
    tile_store_mx<NB, LB>(P, tiles + (q0 & 1) * tile_bytes_mx<LB>());
    __syncthreads();
    for (int l0 = 0; l0 < nq; l0 += DQ) {
#pragma unroll
        for (int v = 0; v < DQ; ++v) {
            const int q = q0 + l0 + v;  // the quad of slot v in this round
            const uint8_t* tile = tiles + (q & 1) * tile_bytes_mx<LB>();
            v8i B[NB];
            uint32_t bs[NB];
            tile_read_mx<NB, LB>(tile, 0, B, bs);
            tile_load_mx<NB>(P, ca, to, q + 1, s_end);  // in flight over the quad's steps
            quadw_steps_mx<MB, NB, DQ, LB, 0>(R, v, c, q + DQ, s_end, tile, B, bs, acc);
            // tile q+1 into the other buffer (its reads ended at the last barrier)
            tile_store_mx<NB, LB>(P, tiles + ((q + 1) & 1) * tile_bytes_mx<LB>());
            __syncthreads();
        }
    }
}

// Ring depth in quads for MB weight blocks and NB activation blocks: about
// 32 loads of 16 bytes per lane in flight (the registers allow two quads
// with two weight blocks and one activation block).
template <int FMT, int MB, int NB>
constexpr int ring_quads() {
    constexpr int per_quad = 4 * (MB + 2 * NB);
    constexpr int budget = MOE_RING_LOADS;
    return budget / per_quad < 1 ? 1 : budget / per_quad;
}

// MXFP8 of 4 consecutive values (part of a 32-value block shared by 8
// consecutive lanes): returns the 4 codes, writes the block's scale code.
__device__ __forceinline__ uint32_t mx_quant4_group8(const float hv[4], uint8_t& scale_out) {
    uint32_t amax = 0;
    int special = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t b = __float_as_uint(hv[c]) & 0x7fffffffu;
        amax = max(amax, b);
        special |= f32_bits_special(b) ? 1 : 0;
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, off, 64));
        special |= __shfl_xor(special, off, 64);
    }
    uint32_t w = 0;
    if (special) {
        scale_out = 0xff;
#pragma unroll
        for (int c = 0; c < 4; ++c) w |= (((__float_as_uint(hv[c]) >> 24) & 0x80u) | 0x7fu) << (8 * c);
    } else {
        const int shared = mx_shared_exp(amax);
        scale_out = (uint8_t)(shared + 127);
        const float f = exp2i(-shared);
        w = e4m3x2_sat(hv[0] * f, hv[1] * f) | (e4m3x2_sat(hv[2] * f, hv[3] * f) << 16);
    }
    return w;
}


// ---- gate_up ----------------------------------------------------------------
// Item = (slot, 32*GMB output columns, K split).  Waves 0/1 stream the gate
// rows of the two halves of the columns, waves 2/3 the matching up rows
// (rows I + ...); each wave owns GMB blocks of 16 rows.  FUSED (one split):
// SwiGLU + MXFP8 requant in the epilogue; h rows are bucket positions
// (routed) or token rows (dense).  Otherwise fp32 partials part[split][row][2I]
// (already multiplied by the NVFP4 row factor).

// 16-row weight blocks per wave in gate_up: two (four: decode 269 -> 296
// us), or one when a two-block grid would not reach one workgroup per CU
// (verify: 26.0 -> 24.8 us alone, tiny 9.1 -> 7.7; decode, whose grid is far
// larger, with one: 269 -> 347 us).  Output columns per workgroup: 32 * blocks.
constexpr int kGateMB = 2, kGateMBSmall = 1;

// Main workgroups [0, n2) take items of a second job J2 of the same format
// (the FP4 shared expert riding along the routed experts; first, so its few
// long items do not trail the launch), [n2, nmain) items of job J0; the rest
// of the grid runs a bf16 shared-expert stage (before or after them).  PR: rows per pass, 32 (two 16-row N-blocks) or 16
// (one: at 16 or fewer token rows no expert has more, and the smaller tiles
// and registers let a third workgroup onto each CU).
template <int FMT, bool FUSED, int GMB, int PR>
__global__ __launch_bounds__(kThreads, kNVW<FMT> ? MOE_NV_MINB : MOE_MIN_BLOCKS) void k_gate_up(
    StreamJob J0, uint8_t* __restrict__ h_q0, uint8_t* __restrict__ h_s0, float* __restrict__ part, int nmain,
    Bf16Side side, int stage, StreamJob J2, uint8_t* __restrict__ h_q2, uint8_t* __restrict__ h_s2, int n2) {
    // A bf16 shared-expert stage riding along takes the workgroups after the
    // main items, or, when the main items need more than one round of resident
    // workgroups (over 768), the first ones: placed last they ran in the
    // launch's tail (skew 203.1 -> 200.8 us per step); within one round they
    // stay last, where they do not take the first issue slots from the routed
    // items (verify, 512 items and 112 riders: 59.8 -> 60.5 us with them first).
    const int nside = (int)gridDim.x - nmain;
    const bool side_first = nmain > 768;
    const int sb = side_first ? (int)blockIdx.x : (int)blockIdx.x - nmain;
    if (sb >= 0 && sb < nside) {
        bf16_side_block(side, stage, sb);
        return;
    }
    const int b0 = side_first ? (int)blockIdx.x - nside : (int)blockIdx.x;
    const bool second = b0 < n2;  // uniform
    const StreamJob& J = second ? J2 : J0;
    uint8_t* __restrict__ h_q = second ? h_q2 : h_q0;
    uint8_t* __restrict__ h_s = second ? h_s2 : h_s0;
    const int bid = second ? b0 : b0 - n2;
    const int I = J.N / 2, K = J.K;
    constexpr int GCOLS = 32 * GMB;  // output columns per workgroup
    const int ks = bid % J.splits;
    int slot, blk;
    item_of(J, bid / J.splits, J.nblk, slot, blk);
    Tokens tk;
    __shared__ int s_list[kIdsPairs], s_tok[kIdsPairs];
    if (!resolve_item(J, slot, tk, s_list, s_tok)) return;
    if (J.r_act && blk == 0 && ks == 0) {  // one workgroup per slot records it for the down launch
        const int t = threadIdx.x;
        for (int u = t; u < tk.n; u += kThreads) {
            J.r_bkt[tk.base + u] = s_list[u];
            if (J.r_yrec) J.r_yrec[s_list[u]] = ygroup_rec(tk.base, tk.n, u, K);
        }
        if (t == 0) {
            J.r_act[slot] = tk.e;
            J.r_off[slot] = tk.base;
            if (slot == 0) {
                *J.r_na = tk.na;
                J.r_off[tk.na] = J.M * J.k;
            }
        }
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    const int half = (wave & 1) * (16 * GMB);  // column offset of the wave within the item
    const int col0 = blk * GCOLS + half;       // first output column of the wave
    int wblk[GMB];  // first W13 row of each of the wave's 16-row blocks
#pragma unroll
    for (int mb = 0; mb < GMB; ++mb) wblk[mb] = (wave >> 1) * I + col0 + 16 * mb;
    const int k0 = ks * J.span;
    const int s0 = k0 / 128, nst = min(J.span, K - k0) / 128;
    const float gs = kNVW<FMT> ? J.gscale[tk.e] : 1.0f;
    // NVFP4 activations: accumulator factor (activation global x weight
    // global) and the global of the h written
    const float fa4 = kA4<FMT> ? act_global(J, tk.e) * gs : 0.0f;
    const float hg4 = kA4<FMT> ? out_global(J, tk.e) : 0.0f;

    // fused epilogue: gate [0, GCOLS), up [GCOLS, 2*GCOLS) per row.  NVFP4 keeps
    // the activation tiles of two quads in the same LDS: the epilogue runs
    // after the pass's last barrier, when no wave reads a tile any more.
    static_assert(PR == 16 || PR == 32, "passes of one or two 16-row N-blocks");
    constexpr int NBX = PR / 16;
    constexpr int kGBytes = PR * (2 * GCOLS + 1) * 4;
    constexpr int kTileLds = kNVW<FMT> ? 2 * tile_bytes_h<NBX>() : 2 * tile_bytes_mx<NBX>();
    constexpr int kLdsBytes = kTileLds > kGBytes ? kTileLds : kGBytes;
    __shared__ __align__(16) uint8_t sLds[kLdsBytes];
    float(*sG)[2 * GCOLS + 1] = reinterpret_cast<float(*)[2 * GCOLS + 1]>(sLds);
    __shared__ int s_smax[PR];

    for (int t0 = 0; t0 < tk.n; t0 += PR) {
        const int npass = min(PR, tk.n - t0);
        const int arow0 = tk.base + t0;
        // token-ordered activations: gather the pass's rows (tokens resolved
        // with the slot, or read from the bucket here)
        const int* src = nullptr;
        if (J.a_tok) {
            if (J.ids) {
                src = s_tok + t0;
            } else {
                __syncthreads();  // the previous pass's reads of s_tok are done
                if ((int)threadIdx.x < npass) s_tok[threadIdx.x] = J.bucket[arow0 + threadIdx.x] / J.k;
                __syncthreads();
                src = s_tok;
            }
        }
        v4f acc[GMB][2];
        int smax[2] = {0, 0};
        // NB = 2 only where a pass can hold two N-blocks (the NB = 1 code is
        // written out for both kernels so each compiles as its own)
        if (NBX > 1 && npass > 16) {
            int sm[2];
            constexpr int NB2 = NBX > 1 ? 2 : 1;
            if constexpr (kNVW<FMT>)
                stream_pass_lds<GMB, NB2, MOE_NV_DQ, kA4<FMT>, NBX>(J, tk.e, wblk, arow0, npass, src, s0, nst,
                                                               reinterpret_cast<int(&)[NB2]>(sm), acc, sLds, s_smax);
            else {  // MXFP4: the activation tile in LDS (measured faster from one row per pass up)
                stream_pass_lds_mx<GMB, NB2, MOE_MX_DQ, NBX>(J, tk.e, wblk, arow0, npass, src, s0, nst, acc, sLds);
                sm[0] = sm[1] = 0;
            }
            smax[0] = sm[0];
            smax[1] = sm[1];
        } else {
            int sm[1];
            if constexpr (kNVW<FMT>)
                stream_pass_lds<GMB, 1, MOE_NV_DQ, kA4<FMT>, NBX>(J, tk.e, wblk, arow0, npass, src, s0, nst, sm, acc,
                                                                  sLds, s_smax);
            else {
                stream_pass_lds_mx<GMB, 1, MOE_MX_DQ, NBX>(J, tk.e, wblk, arow0, npass, src, s0, nst, acc, sLds);
                sm[0] = 0;
            }
            smax[0] = sm[0];
        }
        if constexpr (FUSED) {
#pragma unroll
            for (int mb = 0; mb < GMB; ++mb) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int t = 16 * j + i;
                    if (t < npass) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sG[t][(wave >> 1) * GCOLS + half + 16 * mb + 4 * g + r] = acc[mb][j][r];
                    }
                }
            }
            if (FMT == kFmtNV && wave == 0 && g == 0) {
                s_smax[i] = smax[0];
                s_smax[16 + i] = smax[1];
            }
            __syncthreads();
            // SwiGLU + MXFP8 requant: 8 lanes per 32-column block, 4 columns each
            // (whole waves take part in every round, the row check is per lane).
            for (int idx = threadIdx.x; idx < PR * (GCOLS / 4); idx += kThreads) {
                const int t = idx / (GCOLS / 4), q = idx % (GCOLS / 4);
                float hv[4];
                float fac = 1.0f;
                if (FMT == kFmtNV && t < npass) fac = nv_row_factor(s_smax[t], gs);
                if (kA4<FMT>) fac = fa4;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int col = 4 * q + c;
                    float gt = 0.f, up = 0.f;
                    if (t < npass) {
                        gt = sG[t][col] * fac;
                        up = sG[t][GCOLS + col] * fac;
                    }
                    hv[c] = swiglu(gt, up, J.limit);
                }
                uint8_t sc;
                if constexpr (kA4<FMT>) {
                    // NVFP4 h: 4 lanes per 16-column block, 2 code bytes per lane
                    const uint32_t codes = nvfp4_quant4_lanes4(hv, hg4, sc);
                    if (t < npass) {
                        const size_t orow = (size_t)(arow0 + t);
                        const int col = blk * GCOLS + 4 * q;
                        *reinterpret_cast<uint16_t*>(h_q + orow * (I / 2) + col / 2) = (uint16_t)codes;
                        if ((q & 3) == 0) h_s[orow * (I / 16) + col / 16] = sc;
                    }
                } else {
                    const uint32_t codes = mx_quant4_group8(hv, sc);
                    if (t < npass) {
                        const size_t orow = (size_t)(arow0 + t);
                        *reinterpret_cast<uint32_t*>(h_q + orow * I + blk * GCOLS + 4 * q) = codes;
                        if ((q & 7) == 0) h_s[orow * (I / 32) + blk * (GCOLS / 32) + (q >> 3)] = sc;
                    }
                }
            }
            __syncthreads();
        } else {
#pragma unroll
            for (int mb = 0; mb < GMB; ++mb) {
                const int colw = (wave >> 1) * I + col0 + 16 * mb + 4 * g;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int t = 16 * j + i;
                    if (t < npass) {
                        v4f v = acc[mb][j];
                        if (FMT == kFmtNV) v = v * nv_row_factor(smax[j], gs);
                        if (kA4<FMT>) v = v * fa4;
                        *reinterpret_cast<v4f*>(part + ((size_t)ks * J.out_rows + arow0 + t) * (2 * I) + colw) = v;
                    }
                }
            }
        }
    }
}

// Sum of the split partials in split order, SwiGLU, MXFP8 requant of h.
// Thread = (row, 4 columns); 8 consecutive threads share a 32-column block.
__global__ __launch_bounds__(kThreads) void k_swiglu_quant(const float* __restrict__ part, int splits, int rows,
                                                           int I, uint8_t* __restrict__ h_q,
                                                           uint8_t* __restrict__ h_s, float limit) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;
    const int q8 = idx & 7, blk = idx >> 3;
    const int cbs = I / 32;
    const int row = blk / cbs, cb = blk - row * cbs;
    if (row >= rows) return;  // whole 8-lane groups leave together
    const int col = cb * 32 + 4 * q8;
    v4f gt = v4f{0.f, 0.f, 0.f, 0.f}, up = v4f{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
        const float* pr = part + ((size_t)s * rows + row) * (2 * I);
        gt += *reinterpret_cast<const v4f*>(pr + col);
        up += *reinterpret_cast<const v4f*>(pr + I + col);
    }
    float hv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) hv[c] = swiglu(gt[c], up[c], limit);
    uint8_t sc;
    const uint32_t codes = mx_quant4_group8(hv, sc);
    *reinterpret_cast<uint32_t*>(h_q + (size_t)row * I + col) = codes;
    if (q8 == 0) h_s[(size_t)row * cbs + cb] = sc;
}

// ---- down along K (K above one quad) ------------------------------------------
// Item = (slot, 64*MB output features); wave w owns MB blocks of 16 features.
// Activations are h rows in bucket order; the output row of bucket position b
// is its pair id bucket[b] (the token row for a dense expert).

// 16-row weight blocks per wave in down along K: two, with two quads of
// weights in flight.  Four blocks (one quad in flight, the activation tile
// serving twice the weight rows) measured slower once y of 384 rows is
// written non-temporally: wide down 342 us with two against 359 with four,
// decode 137 against 140.  NVFP4 two (four would spill: its dequantization
// needs registers).
#ifndef MOE_DOWN_MB_WIDE
#define MOE_DOWN_MB_WIDE 2
#endif
constexpr int kDownMBWide = MOE_DOWN_MB_WIDE, kDownMB = 2;

// y of at least this many bytes is written with non-temporal stores (NTY).
// Measured at 384 rows (88 MB of y): the cached stores left y's lines dirty
// in the caches and their write-back landed in the next step's gate_up
// (634.8 -> 613.6 us with NTY, the finalize 21.0 -> 24.6 us: y comes from
// HBM); at 16 or fewer rows (y of 2-8 MB) the finalize's cache hits win.
#ifndef MOE_NT_Y_BYTES
#define MOE_NT_Y_BYTES (32u << 20)
#endif

template <int FMT, int MB, bool NTY, int PR>
__global__ __launch_bounds__(kThreads, MOE_MIN_BLOCKS) void k_down(StreamJob J0, float* __restrict__ y0, StreamJob J2,
                                                                   float* __restrict__ y2, int n2) {
    // workgroups [0, n2) take items of a second job J2 (first: its few long
    // items would otherwise trail the launch), [n2, nmain) items of J0.  PR:
    // rows per pass, as in k_gate_up
    static_assert(PR == 16 || PR == 32, "passes of one or two 16-row N-blocks");
    constexpr int NBX = PR / 16;
    const bool second = (int)blockIdx.x < n2;  // uniform
    const StreamJob& J = second ? J2 : J0;
    float* __restrict__ y = second ? y2 : y0;
    const int bid = second ? (int)blockIdx.x : (int)blockIdx.x - n2;
    const int H = J.N, I = J.K;
    constexpr int RB = 64 * MB;
    int slot, blk;
    item_of(J, bid, J.nblk, slot, blk);
    Tokens tk;
    __shared__ int s_list[kIdsPairs], s_tok[kIdsPairs];
    if (!resolve_item(J, slot, tk, s_list, s_tok)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    const int f0 = blk * RB + wave * (16 * MB);
    int wblk[MB];  // first W2 row of each of the wave's 16-row blocks
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) wblk[mb] = f0 + 16 * mb;
    const int nst = I / 128;
    const float gs = kNVW<FMT> ? J.gscale[tk.e] : 1.0f;
    const float fa4 = kA4<FMT> ? act_global(J, tk.e) * gs : 0.0f;  // NVFP4 h: its global x the weights'
    // MXFP4: the h tiles in LDS (the NVFP4 formats stream h from registers)
    __shared__ __align__(16) uint8_t sTile[FMT == kFmtMX ? 2 * tile_bytes_mx<NBX>() : 16];
    constexpr int kDownDQ = MB > 2 ? MOE_MX_DOWN_DQ : MOE_MX_DQ;  // ring quads the registers allow

    for (int t0 = 0; t0 < tk.n; t0 += PR) {
        const int npass = min(PR, tk.n - t0);
        const int arow0 = tk.base + t0;
        // output rows of the lane's activation rows: loaded before the ring so
        // they return first
        int orow[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = 16 * j + i;
            orow[j] = t < npass ? (J.dense ? arow0 + t : J.ids ? s_list[t0 + t] : J.bucket[arow0 + t]) : 0;
        }
        v4f acc[MB][2];
        int smax[2] = {0, 0};
        constexpr int NB2 = NBX > 1 ? 2 : 1;  // NB = 2 only where a pass can hold two N-blocks
        if constexpr (FMT == kFmtMX) {  // the workgroup shares the h tile in LDS
            if (NBX > 1 && npass > 16)
                stream_pass_lds_mx<MB, NB2, kDownDQ, NBX>(J, tk.e, wblk, arow0, npass, nullptr, 0, nst, acc, sTile);
            else
                stream_pass_lds_mx<MB, 1, kDownDQ, NBX>(J, tk.e, wblk, arow0, npass, nullptr, 0, nst, acc, sTile);
        } else if (NBX > 1 && npass > 16) {
            int sm[2];
            stream_pass<FMT, MB, NB2, ring_quads<FMT, MB, NB2>(), 4>(J, tk.e, wblk, arow0, npass, nullptr, 0, nst,
                                                                     reinterpret_cast<int(&)[NB2]>(sm), acc);
            smax[0] = sm[0];
            smax[1] = sm[1];
        } else {
            int sm[1];
            stream_pass<FMT, MB, 1, ring_quads<FMT, MB, 1>(), 4>(J, tk.e, wblk, arow0, npass, nullptr, 0,
                                                                                 nst, sm, acc);
            smax[0] = sm[0];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = 16 * j + i;
            if (t < npass) {
                // grouped y: block j of the pass is one group of min(16, npass - 16 j) rows
                const int grows = min(kYGroupRows, npass - 16 * j);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    v4f v = acc[mb][j];
                    if (FMT == kFmtNV) v = v * nv_row_factor(smax[j], gs);
                    if (kA4<FMT>) v = v * fa4;
                    const int col = f0 + 16 * mb + 4 * g;
                    const size_t yo = J.ygrp ? (size_t)(arow0 + 16 * j) * H + (size_t)(col / kYBlockCols) * (grows * kYBlockCols) +
                                                   i * kYBlockCols + col % kYBlockCols
                                             : (size_t)orow[j] * H + col;
                    v4f* dst = reinterpret_cast<v4f*>(y + yo);
                    if constexpr (NTY)
                        __builtin_nontemporal_store(v, dst);
                    else
                        *dst = v;
                }
            }
        }
    }
}

// The S steps of one 16-row block in down-by-rows (step U at a time; the
// MFMA's scale byte selects are immediates).
template <int FMT, int S, int D, int U>
__device__ __forceinline__ void rows_steps(v4f& acc, const v4i (&wa)[D][S], const uint32_t (&wsc)[D][FMT == kFmtMX ? 1 : 2],
                                           int d, const v4i (&b)[S][2], const uint32_t (&bs)[S],
                                           const v8h (&B16)[kNVW<FMT> ? S : 1][4], int g) {
    if constexpr (U < S) {
        const v4i a = wa[d][U];
        if constexpr (FMT == kFmtMX) {
            const v8i A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
            const v8i Bm = {b[U][0].x, b[U][0].y, b[U][0].z, b[U][0].w, b[U][1].x, b[U][1].y, b[U][1].z, b[U][1].w};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bm, acc, 4, 0, U, (int)wsc[d][0], 0,
                                                                   (int)(bs[U] >> (8 * g)));
        } else {
            float sv0, sv1;
            v2h m;
            nv_scales2<U & 1>(wsc[d][U >> 1], sv0, sv1, m);
            const v8h A0 = nv_dequant8((uint32_t)a.x, sv0, m[0]);
            const v8h A1 = nv_dequant8((uint32_t)a.y, sv0, m[0]);
            const v8h A2 = nv_dequant8((uint32_t)a.z, sv1, m[1]);
            const v8h A3 = nv_dequant8((uint32_t)a.w, sv1, m[1]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B16[U][0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B16[U][1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A2, B16[U][2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A3, B16[U][3], acc, 0, 0, 0);
        }
        rows_steps<FMT, S, D, U + 1>(acc, wa, wsc, d, b, bs, B16, g);
    }
}

// ---- down for a short K: streaming along the output rows ---------------------
// When all of K is one quad (S = K/128 <= 4 steps) there is nothing to stream
// along K, so an item streams its weight rows instead: each wave converts its
// pass's activation rows once and keeps them in registers, keeps D blocks of 16
// weight rows in flight, and writes a block's outputs as soon as its S steps
// are done (stores past the wave's blocks or the pass's rows are dropped by the
// buffer range check, so the loop has no branches).  Item = (slot, run of
// 4 * bpw blocks); wave w takes blocks [w * bpw, (w + 1) * bpw) of the run.
// Passes of 16 activation rows; a later pass reads the item's weights again.
template <int FMT, int S, int D>
__global__ __launch_bounds__(kThreads, MOE_MIN_BLOCKS) void k_down_rows(StreamJob J, float* __restrict__ y) {
    const int H = J.N, K = J.K;
    const int bpw = J.span;
    int slot, item;
    item_of(J, blockIdx.x, J.nblk, slot, item);
    Tokens tk;
    __shared__ int s_list[kIdsPairs], s_tok[kIdsPairs];
    if (!resolve_item(J, slot, tk, s_list, s_tok)) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, g = lane >> 4;
    const int nbr = H / 16;
    const int rb0 = (item * 4 + wave) * bpw;
    const int nb = max(0, min(bpw, nbr - rb0));
    constexpr int SQ = FMT == kFmtMX ? 256 : 512;  // scale bytes per block (one quad)
    const uint32_t wbytes = (uint32_t)H * (K / 2), sbytes = (uint32_t)nbr * SQ;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(J.w + (size_t)tk.e * wbytes, wbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(J.sc + (size_t)tk.e * sbytes, sbytes);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y, (uint32_t)J.out_rows * (uint32_t)H * 4u);
    const float gs = kNVW<FMT> ? J.gscale[tk.e] : 1.0f;
    // activation row bytes: MXFP8 K codes + K/32 scales; NVFP4 K/2 + K/16
    constexpr int kAQd = kA4<FMT> ? 2 : 1, kASd = kA4<FMT> ? 16 : 32;

    for (int t0 = 0; t0 < tk.n; t0 += 16) {
        const int npass = min(16, tk.n - t0);
        const int arow0 = tk.base + t0;
        const bool okr = i < npass;
        const int orow = okr ? (J.dense ? arow0 + i : J.ids ? s_list[t0 + i] : J.bucket[arow0 + i]) : 0;
        // the lane's activation row (column i of the MFMAs), all S steps
        const int AQ = K / kAQd, AS = K / kASd;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(J.a_q + (size_t)arow0 * AQ, (uint32_t)npass * (uint32_t)AQ);
        const __amdgpu_buffer_rsrc_t ras = make_rsrc(J.a_s + (size_t)arow0 * AS, (uint32_t)npass * (uint32_t)AS);
        // NVFP4 h: bytes [16g, +16) of each step's 64 and the dword of the
        // lane's two scale bytes (2g, 2g + 1 of the step's 8)
        const uint32_t va = okr ? (uint32_t)i * AQ + (kA4<FMT> ? 16 : FMT == kFmtMX ? 16 : 32) * g : kOOB;
        const uint32_t vas = okr ? (uint32_t)i * AS + (kA4<FMT> ? 4 * (g >> 1) : 0) : kOOB;
        v4i b[S][2];
        uint32_t bs[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if constexpr (kA4<FMT>) {
                b[s][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, va, 64 * s, 0);
                b[s][1] = v4i{0, 0, 0, 0};
                bs[s] = __builtin_amdgcn_raw_buffer_load_b32(ras, vas, 8 * s, 0);
            } else {
                b[s][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, va, 128 * s, 0);
                b[s][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, va + (FMT == kFmtMX ? 64 : 16), 128 * s, 0);
                bs[s] = __builtin_amdgcn_raw_buffer_load_b32(ras, vas, 4 * s, 0);
            }
        }
        // weight ring: slot d holds one block (S steps and its scale entry)
        v4i wa[D][S];
        uint32_t wsc[D][FMT == kFmtMX ? 1 : 2];
        auto load_block = [&](int d, int blk) {
            const bool ok = blk < nb;
            const uint32_t rb = (uint32_t)(rb0 + blk);
            const uint32_t vw = ok ? rb * S * 1024 + 16 * lane : kOOB;
            const uint32_t vs = ok ? rb * SQ + (SQ / 64) * lane : kOOB;
#pragma unroll
            for (int s = 0; s < S; ++s)
                wa[d][s] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw, 1024 * s, MOE_WEIGHT_AUX);
            if constexpr (FMT == kFmtMX) {
                wsc[d][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs, 0, 0);
            } else {
                const auto sv = __builtin_amdgcn_raw_buffer_load_b64(rs, vs, 0, 0);
                wsc[d][0] = sv[0];
                wsc[d][1] = sv[1];
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d) {
            __builtin_amdgcn_sched_barrier(0);
            load_block(d, d);
        }
        __builtin_amdgcn_sched_barrier(0);
        // activations as MFMA operands: MX keeps the codes; NV converts to f16
        // scaled by 2^(s - smax) with smax the row's largest scale code
        int smax = 0;
        float fac = 1.0f;
        v8h B16[kNVW<FMT> ? S : 1][4];
        if constexpr (kA4<FMT>) {
#pragma unroll
            for (int s = 0; s < S; ++s) act4_to_f16(b[s][0], bs[s], g, B16[s]);
            fac = act_global(J, tk.e) * gs;
        } else if constexpr (FMT == kFmtNV) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t v = bs[s];
                smax = max(smax, (int)max(max(v & 0xffu, (v >> 8) & 0xffu), max((v >> 16) & 0xffu, v >> 24)));
            }
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int sb = (int)((bs[s] >> (8 * g)) & 0xffu);
                const float sf = exp2i(max(sb - smax, -126));
                B16[s][0] = fp8x8_to_f16((uint32_t)b[s][0].x, (uint32_t)b[s][0].y, sf);
                B16[s][1] = fp8x8_to_f16((uint32_t)b[s][0].z, (uint32_t)b[s][0].w, sf);
                B16[s][2] = fp8x8_to_f16((uint32_t)b[s][1].x, (uint32_t)b[s][1].y, sf);
                B16[s][3] = fp8x8_to_f16((uint32_t)b[s][1].z, (uint32_t)b[s][1].w, sf);
            }
            fac = nv_row_factor(smax, gs);
        }
        // y by pair: the lane's row; grouped: the pass is one group of npass rows
        // whose 128-column blocks (eight 16-column weight blocks) are npass rows apart
        const uint32_t ybase = okr ? (J.ygrp ? ((uint32_t)arow0 * (uint32_t)H + (uint32_t)i * kYBlockCols) * 4u
                                             : (uint32_t)orow * (uint32_t)H * 4u) + 16u * g
                                   : kOOB;
        const uint32_t ygs = J.ygrp ? (uint32_t)npass * kYBlockCols * 4u : 8u * 64u;  // bytes per 8 weight blocks
        static_assert(kYBlockCols == 8 * 16, "a y column block is eight 16-row weight blocks");
        for (int b0 = 0; b0 < nb; b0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                __builtin_amdgcn_sched_barrier(0);
                v4f acc = {0.f, 0.f, 0.f, 0.f};
                rows_steps<FMT, S, D, 0>(acc, wa, wsc, d, b, bs, B16, g);
                const int blk = b0 + d;
                const uint32_t cb = (uint32_t)(rb0 + blk);
                const uint32_t vo = blk < nb ? ybase + (cb >> 3) * ygs + (cb & 7u) * 64u : kOOB;
                const v4f v = acc * fac;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), ry, vo, 0, 0);
                load_block(d, blk + D);
            }
        }
    }
}

// ---- host plans -------------------------------------------------------------

// Slot dimension of a launch: the active-expert slots, or a dense job's passes.
int grid_slots(const ExpertJob& j) { return j.dense ? (j.M + kPassRows - 1) / kPassRows : j.slots; }

struct GatePlan {
    int span, splits, nblk;
};

// Weight blocks per wave of a gate_up launch (see kGateMB).
int gate_mb(const ExpertJob& j) {
#ifdef MOE_GATE_MB_FORCE
    return MOE_GATE_MB_FORCE;
#endif
    // one block when a two-block grid would not reach one workgroup per CU, or
    // when it would spill just past one round of resident workgroups (two per
    // CU): then half-size items shorten the tail
    const long items = (long)grid_slots(j) * (j.N_out / (32 * kGateMB));
    return items <= 256 || (items > 512 && items <= 768) ? kGateMBSmall : kGateMB;
}

GatePlan gate_plan(const ExpertJob& j, int gmb) {
    GatePlan p;
    const int K = j.K, steps = K / 128;
    p.nblk = j.N_out / (32 * gmb);
    if (j.a_nvfp4) {  // NVFP4 activations: all of K in one item (the requant needs the expert's h global)
        p.span = K;
        p.splits = 1;
        return p;
    }
    const long items = (long)grid_slots(j) * p.nblk;
    int want = (int)std::max<long>(1, (MOE_STREAM_TARGET_ITEMS + items - 1) / items);
    want = std::min(want, std::max(1, steps / 8));  // at least 8 steps per split
    int sps = (steps + want - 1) / want;             // steps per split: whole quads
    if (sps < steps) sps = (sps + 3) / 4 * 4;
    p.span = 128 * sps;
    p.splits = (steps + sps - 1) / sps;
    return p;
}

StreamJob stream_job(const ExpertJob& j, int N, const uint8_t* a_q, const uint8_t* a_s, int a_rows) {
    StreamJob s;
    s.w = static_cast<const uint8_t*>(j.w.w);
    s.sc = j.w.scales;
    s.gscale = j.w.global_scale;
    s.N = N;
    s.K = j.K;
    s.dense = j.dense ? 1 : 0;
    s.bucket = j.bucket;
    s.active = j.active;
    s.active_offsets = j.active_offsets;
    s.M = j.M;
    s.a_q = a_q;
    s.a_s = a_s;
    s.a_rows = (uint32_t)a_rows;
    s.span = j.K;
    s.splits = 1;
    s.nblk = 1;
    s.out_rows = a_rows;
    s.ids = j.dense ? nullptr : j.ids;
    s.k = j.k;
    s.a_tok = (!j.dense && j.a_tok) ? 1 : 0;
    s.count = j.dense ? nullptr : j.count;
    s.r_act = j.record ? j.record->act : nullptr;
    s.r_off = j.record ? j.record->off : nullptr;
    s.r_na = j.record ? j.record->na : nullptr;
    s.r_bkt = j.record ? j.record->bkt : nullptr;
    s.r_yrec = j.record ? j.record->yrec : nullptr;
    s.ygrp = j.ygroup ? 1 : 0;
    if (s.a_tok) s.a_rows = (uint32_t)j.M;
    s.limit = j.swiglu_limit;
    s.ag = j.a_global;
    s.age = j.a_globals;
    s.hg = j.h_global;
    s.hge = j.h_globals;
    return s;
}

int out_rows_of(const ExpertJob& j) { return j.dense ? j.M : j.M * j.k; }

}  // namespace

size_t gate_up_fp4_partials_bytes(const ExpertJob& job) {
    const int gmb = gate_mb(job);
    const GatePlan p = gate_plan(job, gmb);
    if (p.splits == 1) return 0;
    return align_up((size_t)p.splits * out_rows_of(job) * 2 * job.N_out * sizeof(float));
}

// Rows per pass of a launch: 16 when its jobs have at most 16 token rows (an
// expert gets at most one row per token: one 16-row N-block per pass, with
// half the LDS tiles and fewer registers, so three workgroups fit on a CU;
// measured at 7 rows of NVFP4 activations 85.2 -> 80.8 us per step, decode
// 423 -> 419 us), else 32.
int pass_rows(const ExpertJob& j, const ExpertJob* j2) { return j.M <= 16 && (!j2 || j2->M <= 16) ? 16 : 32; }

// One gate_up launch with the kernel of gmb weight blocks per wave and pr rows per pass.
template <int F, bool FU, int PR>
hipError_t launch_gu_pr(int gmb, dim3 g, hipStream_t stream, const StreamJob& J, uint8_t* h_q, uint8_t* h_s,
                        float* partials, int nmain, const Bf16Side& side, int stage, const StreamJob& J2,
                        uint8_t* hq2, uint8_t* hs2, int n2) {
    if (gmb == kGateMBSmall) {
        hipLaunchKernelGGL((k_gate_up<F, FU, kGateMBSmall, PR>), g, dim3(kThreads), 0, stream, J, h_q, h_s, partials,
                           nmain, side, stage, J2, hq2, hs2, n2);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_gate_up<F, FU, kGateMB, PR>), g, dim3(kThreads), 0, stream, J, h_q, h_s, partials, nmain,
                       side, stage, J2, hq2, hs2, n2);
    return hipGetLastError();
}
template <int F, bool FU>
hipError_t launch_gu(int pr, int gmb, dim3 g, hipStream_t stream, const StreamJob& J, uint8_t* h_q, uint8_t* h_s,
                     float* partials, int nmain, const Bf16Side& side, int stage, const StreamJob& J2, uint8_t* hq2,
                     uint8_t* hs2, int n2) {
    return pr == 16 ? launch_gu_pr<F, FU, 16>(gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2, hq2, hs2, n2)
                    : launch_gu_pr<F, FU, 32>(gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2, hq2, hs2,
                                              n2);
}

hipError_t launch_gate_up_fp4(const ExpertJob& job, const uint8_t* a_q, const uint8_t* a_s, uint8_t* h_q,
                              uint8_t* h_s, float* partials, hipStream_t stream, const Bf16Side& side, int stage,
                              const SecondJob& second) {
    const int gmb = gate_mb(job);
    const GatePlan p = gate_plan(job, gmb);
    const int rows = out_rows_of(job);
    StreamJob J = stream_job(job, 2 * job.N_out, a_q, a_s, rows);
    J.span = p.span;
    J.splits = p.splits;
    J.nblk = p.nblk;
    const int blocks = grid_slots(job) * p.nblk * p.splits;
    const bool mx = job.w.fmt == MOE_FMT_MXFP4;
    // a second job of the same formats rides along when both run over all of K
    StreamJob J2 = J;
    int n2 = 0;
    if (second.job) {
        const ExpertJob& j2 = *second.job;
        if (p.splits == 1 && j2.w.fmt == job.w.fmt && j2.a_nvfp4 == job.a_nvfp4) {
            J2 = stream_job(j2, 2 * j2.N_out, second.a_q, second.a_s, out_rows_of(j2));
            J2.nblk = j2.N_out / (32 * gmb);  // span = K, one split
            n2 = grid_slots(j2) * J2.nblk;
        } else {
            hipError_t e = launch_gate_up_fp4(j2, second.a_q, second.a_s, second.h_q, second.h_s, second.partials,
                                              stream);
            if (e != hipSuccess) return e;
        }
    }
    const int extra = stage == kBf16None ? 0 : side.blocks;
    const dim3 g(blocks + n2 + extra);
    uint8_t* hq2 = n2 ? second.h_q : h_q;
    uint8_t* hs2 = n2 ? second.h_s : h_s;
    const int nmain = blocks + n2;
    const int pr = pass_rows(job, n2 ? second.job : nullptr);
    if (p.splits == 1) {
        if (job.a_nvfp4)
            return launch_gu<kFmtNV4, true>(pr, gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2, hq2, hs2,
                                            n2);
        if (mx)
            return launch_gu<kFmtMX, true>(pr, gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2, hq2, hs2,
                                           n2);
        return launch_gu<kFmtNV, true>(pr, gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2, hq2, hs2,
                                       n2);
    }
    hipError_t e = mx ? launch_gu<kFmtMX, false>(pr, gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2,
                                                 hq2, hs2, n2)
                      : launch_gu<kFmtNV, false>(pr, gmb, g, stream, J, h_q, h_s, partials, nmain, side, stage, J2,
                                                 hq2, hs2, n2);
    if (e != hipSuccess) return e;
    const int threads = rows * (job.N_out / 32) * 8;
    hipLaunchKernelGGL(k_swiglu_quant, dim3((threads + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                       partials, p.splits, rows, job.N_out, h_q, h_s, job.swiglu_limit);
    return hipGetLastError();
}

// Down by rows (K of at most one quad): blocks per wave and items per slot so
// that about two workgroups per CU stream runs of equal length.
template <int FMT, int S>
hipError_t launch_down_rows_s(StreamJob J, int slots, float* y, hipStream_t stream) {
    constexpr int D = 4;  // blocks in flight per wave (deeper rings measured slower)
    const int nbr = J.N / 16;
    int items = std::max(1, std::min(MOE_ROWS_TARGET_WGS / std::max(1, slots), nbr / (4 * D)));
    // a run short enough that an expert with many passes still spreads out
    constexpr int max_bpw = MOE_ROWS_MAX_KB / S;
    items = std::max(items, (nbr + 4 * max_bpw - 1) / (4 * max_bpw));
    const int bpw = (nbr + 4 * items - 1) / (4 * items);
    items = (nbr + 4 * bpw - 1) / (4 * bpw);
    J.span = bpw;
    J.nblk = items;
    const int nmain = slots * items;
    hipLaunchKernelGGL((k_down_rows<FMT, S, D>), dim3(nmain), dim3(kThreads), 0, stream, J, y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_down_rows(const StreamJob& J, int slots, float* y, hipStream_t stream) {
    switch (J.K / 128) {
        case 1: return launch_down_rows_s<FMT, 1>(J, slots, y, stream);
        case 2: return launch_down_rows_s<FMT, 2>(J, slots, y, stream);
        case 3: return launch_down_rows_s<FMT, 3>(J, slots, y, stream);
        default: return launch_down_rows_s<FMT, 4>(J, slots, y, stream);
    }
}

template <int FMT, int MB, bool NTY>
hipError_t launch_down_k(int pr, dim3 g, hipStream_t stream, const StreamJob& J, float* y, const StreamJob& J2,
                         float* y2, int n2) {
    if (pr == 16)
        hipLaunchKernelGGL((k_down<FMT, MB, NTY, 16>), g, dim3(kThreads), 0, stream, J, y, J2, y2, n2);
    else
        hipLaunchKernelGGL((k_down<FMT, MB, NTY, 32>), g, dim3(kThreads), 0, stream, J, y, J2, y2, n2);
    return hipGetLastError();
}

hipError_t launch_down_fp4(const ExpertJob& job, const uint8_t* h_q, const uint8_t* h_s, float* y,
                           hipStream_t stream, const SecondDown& second) {
    StreamJob J = stream_job(job, job.N_out, h_q, h_s, out_rows_of(job));
    // a second job rides along when both stream along K with the same format
    const bool fold = second.job && job.K > 512 && second.job->K > 512 && second.job->w.fmt == job.w.fmt &&
                      second.job->a_nvfp4 == job.a_nvfp4;
    if (second.job && !fold) {
        hipError_t e = launch_down_fp4(*second.job, second.h_q, second.h_s, second.y, stream);
        if (e != hipSuccess) return e;
    }
    if (job.K <= 512)  // all of K in one quad: stream along the rows
        return job.a_nvfp4                 ? launch_down_rows<kFmtNV4>(J, grid_slots(job), y, stream)
               : job.w.fmt == MOE_FMT_MXFP4 ? launch_down_rows<kFmtMX>(J, grid_slots(job), y, stream)
                                            : launch_down_rows<kFmtNV>(J, grid_slots(job), y, stream);
    const bool mx = job.w.fmt == MOE_FMT_MXFP4;
    const bool wide = mx && job.N_out % (64 * kDownMBWide) == 0;
    const int dmb = wide ? kDownMBWide : kDownMB;
    J.nblk = job.N_out / (64 * dmb);
    const int n1 = grid_slots(job) * J.nblk;
    StreamJob J2 = J;
    int n2 = 0;
    if (fold) {
        const ExpertJob& j2 = *second.job;
        J2 = stream_job(j2, j2.N_out, second.h_q, second.h_s, out_rows_of(j2));
        J2.nblk = j2.N_out / (64 * dmb);
        n2 = grid_slots(j2) * J2.nblk;
    }
    float* y2 = fold ? second.y : y;
    const int nmain = n1 + n2;
    const dim3 g(nmain), b(kThreads);
    const bool nty = (size_t)out_rows_of(job) * job.N_out * sizeof(float) >= MOE_NT_Y_BYTES;
    const int pr = pass_rows(job, fold ? second.job : nullptr);
    if (wide)
        return nty ? launch_down_k<kFmtMX, kDownMBWide, true>(pr, g, stream, J, y, J2, y2, n2)
                   : launch_down_k<kFmtMX, kDownMBWide, false>(pr, g, stream, J, y, J2, y2, n2);
    if (mx)
        return nty ? launch_down_k<kFmtMX, kDownMB, true>(pr, g, stream, J, y, J2, y2, n2)
                   : launch_down_k<kFmtMX, kDownMB, false>(pr, g, stream, J, y, J2, y2, n2);
    if (job.a_nvfp4)
        return nty ? launch_down_k<kFmtNV4, kDownMB, true>(pr, g, stream, J, y, J2, y2, n2)
                   : launch_down_k<kFmtNV4, kDownMB, false>(pr, g, stream, J, y, J2, y2, n2);
    return nty ? launch_down_k<kFmtNV, kDownMB, true>(pr, g, stream, J, y, J2, y2, n2)
               : launch_down_k<kFmtNV, kDownMB, false>(pr, g, stream, J, y, J2, y2, n2);
}

}  // namespace moe
