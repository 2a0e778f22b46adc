// gate_proj.hip -- the RG-LRU gate projections on MFMA: two 16-block
// block-diagonal linear layers in front of the gated scan, and their adjoint.
//
// Page 'Griffin 第 4、5 节 H800 对照协议', 'RG-LRU 的固定方程': both gates are
// computed by 16-block block-diagonal linear layers; training runs them in
// BF16 autocast.  With Db = D/16 and block i covering channels
// [i Db, (i+1) Db), weights stored [16, Db, Db] as (block, output, input):
//   l[t, i Db + o] = b[i Db + o] + sum_k W[i][o][k] x[t, i Db + k]
// for l = l^x (W_x, b_x) and l = l^a (W_a, b_a), rounded to BF16 for the scan.
// Adjoint for the logit cotangents dl^x, dl^a produced by the scan backward:
//   dx[t, i Db + k] += sum_o (W_x[i][o][k] dl^x + W_a[i][o][k] dl^a)[t, i Db + o]
//   dW[i][o][k] = sum_t dl[t, i Db + o] x[t, i Db + k],  db = sum_t dl.
//
// All products run on v_mfma_f32_16x16x32_bf16: lane l supplies eight
// consecutive reduction elements of row l%16 of A and of column l%16 of B
// (group l/16 of the 32) and receives D[4(l/16)+r][l%16], r = 0..3.  A and
// B use the same assignment of reduction indices to (lane group, slot), so
// the sum is the full 32-term dot product whatever order the unit takes.
// FP32 cotangents are split exactly into three BF16 terms (hi + mid + lo =
// the FP32 value: each step keeps the next 8 significand bits), and each
// product with a BF16 operand is then three BF16 products with FP32
// accumulation -- the same exact products as an FP32 multiply, at the BF16
// matrix-core rate.
//
// The work is HBM-bound (a few dozen flops per byte moved), so the kernels
// are shaped for bytes in flight: the forward and dx hold their weights in
// registers as matrix fragments for the life of a workgroup, token tiles are
// requested up to two tiles ahead into registers with branch-free loads
// (so the wait for one tile never covers the tiles behind it), and the grid
// runs the 16 blocks fastest, so that neighbouring workgroups read whole
// token rows.  Output rows of the forward and of dx are permuted inside each
// pair of 16-channel tiles (row i of half h is channel 8 (i/4) + 4 h + i%4
// of the pair) so that every lane ends with eight consecutive channels of
// one token and writes them as one 16-byte store.  dW reduces over tokens:
// its tiles stay in their natural layout in LDS and its fragments come from
// the gfx950 transposing LDS read.
#include "common.hpp"

namespace lrs {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int TT = 64;    // tokens per tile
constexpr int XPAD = 8;   // BF16 elements of LDS row padding (rows of 16-byte fragment reads)
constexpr int FPAD = 4;   // FP32 elements of LDS row padding

#ifndef LRS_GP_TARGET_WG
#define LRS_GP_TARGET_WG 1024   // forward / dx workgroups aimed for
#endif
#ifndef LRS_GP_DW_RANGE
#define LRS_GP_DW_RANGE 2048    // tokens per dW partial sum
#endif
#ifndef LRS_GP_ADJ_FUSED
#define LRS_GP_ADJ_FUSED 1      // BF16 adjoint as one pass (dx and dW from shared tiles)
#endif

template <int MT>
struct Geo {
    static constexpr int Db = 16 * MT;
    static constexpr int P = (MT + 1) / 2;   // pairs of 16-channel tiles
    static constexpr int KS = (MT + 1) / 2;  // 32-wide reduction steps over Db
    static constexpr bool ODD = (MT & 1) != 0;  // last pair / step half used
};

__device__ __forceinline__ v4f mfma(v4u a, v4u b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                   0, 0);
}
__device__ __forceinline__ v4u ld16(const void* p) { return *reinterpret_cast<const v4u*>(p); }
__device__ __forceinline__ void st16(void* p, v4u v) { *reinterpret_cast<v4u*>(p) = v; }
__device__ __forceinline__ v4u zero4() { return v4u{0u, 0u, 0u, 0u}; }

// channel (within the block) of fragment row i, half h, of pair p
__device__ __forceinline__ int pair_chan(int p, int i, int h) { return 32 * p + 8 * (i >> 2) + 4 * h + (i & 3); }

// Exact split of eight FP32 values into BF16 hi + mid + lo (truncations: the
// residual after each step is exact in FP32 and holds at most 16, then 8,
// significant bits).
__device__ __forceinline__ void split3(v4u a, v4u b, v4u& hi, v4u& mid, v4u& lo) {
    const uint32_t f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        h[j] = f[j] & 0xffff0000u;
        const float r1 = __uint_as_float(f[j]) - __uint_as_float(h[j]);
        m[j] = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(m[j]);
        l[j] = __float_as_uint(r2) & 0xffff0000u;
    }
#define GP_PK(v, j) (((v)[2 * (j)] >> 16) | (v)[2 * (j) + 1])
    hi = v4u{GP_PK(h, 0), GP_PK(h, 1), GP_PK(h, 2), GP_PK(h, 3)};
    mid = v4u{GP_PK(m, 0), GP_PK(m, 1), GP_PK(m, 2), GP_PK(m, 3)};
    lo = v4u{GP_PK(l, 0), GP_PK(l, 1), GP_PK(l, 2), GP_PK(l, 3)};
#undef GP_PK
}

// Scheduling fence: nothing moves across it.  The loads of successive
// prefetch stages stay in stage order (so the wait for one stage never
// covers the stages behind it) and work on a prefetched tile stays after the
// barrier that precedes its use.
#ifndef LRS_GP_FENCE
#define LRS_GP_FENCE 1
#endif
#ifndef LRS_GP_FWD_NT
#define LRS_GP_FWD_NT 1
#endif
// forward logits staged through LDS and written as whole token rows (each
// 128-byte line by one store instruction) instead of by the four lanes that
// hold a token's channels of one pair
#ifndef LRS_GP_FWD_STAGE
#define LRS_GP_FWD_STAGE 1
#endif
__device__ __forceinline__ void sched_fence() {
    if (LRS_GP_FENCE) __builtin_amdgcn_sched_barrier(0);
}

// element j (0..3) of four consecutive BF16 values held as (lo word, hi word)
__device__ __forceinline__ uint32_t bf16_at(uint2 v, int j) {
    return ((j < 2 ? v.x : v.y) >> ((j & 1) ? 16 : 0)) & 0xffffu;
}

// dst[c][t] = src[t][c] for a [T, C] BF16 block (row stride gs), dst rows of
// TS elements; each thread moves 4x4 blocks.
__device__ __forceinline__ void stage_transposed_bf16(uint16_t* dst, int TS, const uint16_t* src, size_t gs, int T,
                                                      int C, int nthreads) {
    const int qc = C / 4;
    for (int q = threadIdx.x; q < (T / 4) * qc; q += nthreads) {
        const int a = q / qc, bq = q - a * qc;
        uint2 v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = *reinterpret_cast<const uint2*>(src + (size_t)(4 * a + r) * gs + 4 * bq);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint2*>(dst + (size_t)(4 * bq + j) * TS + 4 * a) =
                make_uint2(bf16_at(v[0], j) | (bf16_at(v[1], j) << 16), bf16_at(v[2], j) | (bf16_at(v[3], j) << 16));
    }
}

// workgroup token ranges of the forward and dx kernels: whole tiles, about
// LRS_GP_TARGET_WG workgroups over the 16 blocks
int stream_range(int BL) {
    const int64_t tiles = ceil_div(BL, TT);
    const int64_t per = std::max<int64_t>(1, ceil_div(tiles * 16, LRS_GP_TARGET_WG));
    return (int)(per * TT);
}

// ------------------------------------------------------------- forward ---
// grid (16 blocks, ranges).  l^T[o][t] = W[o][k] x^T[k][t]: A = W rows
// (registers), B = x rows (LDS).  Wave w owns unit (gate w / P, pair w % P)
// and all tokens; waves past 2 P only help stage tiles.
template <int MT>
constexpr int fwd_waves() {
    return 2 * Geo<MT>::P > 4 ? 2 * Geo<MT>::P : 4;
}

template <int MT>
__global__ __launch_bounds__(64 * fwd_waves<MT>()) void gate_proj_fwd_kernel(
    int BL, int D, int range, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_x,
    const float* __restrict__ b_x, const uint16_t* __restrict__ w_a, const float* __restrict__ b_a,
    uint16_t* __restrict__ lx, uint16_t* __restrict__ la) {
    using G = Geo<MT>;
    constexpr int Db = G::Db, NW = fwd_waves<MT>(), NT = 64 * NW, RS = Db + XPAD;
    constexpr int CPR = Db / 8, NCH = TT * CPR, S = (NCH + NT - 1) / NT;  // 16-byte chunks
    constexpr bool STAGE = LRS_GP_FWD_STAGE != 0;
    extern __shared__ uint16_t gp_lds[];
    uint16_t* const buf0 = gp_lds;
    uint16_t* const buf1 = gp_lds + TT * RS;
    uint16_t* const sout = gp_lds + 2 * TT * RS;  // STAGE: logits [2 gates][TT][RS]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
    const int blk = blockIdx.x;
    const size_t tr0 = (size_t)blockIdx.y * range, tr1 = min((size_t)BL, tr0 + range);
    const int ntile = (int)((tr1 - tr0 + TT - 1) / TT);
    const bool has_unit = wave < 2 * G::P;
    const int g = has_unit ? wave / G::P : 0, p = has_unit ? wave % G::P : 0;
    const uint16_t* W = (g ? w_a : w_x) + (size_t)blk * Db * Db;
    const int c0 = 32 * p + 8 * grp;            // first of this lane's eight output channels
    const bool cv = has_unit && c0 + 8 <= Db;

    v4u wf[2][G::KS];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int o = pair_chan(p, col, h);
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const int k0 = 32 * ks + 8 * grp;
            wf[h][ks] = (has_unit && o < Db && k0 < Db) ? ld16(W + (size_t)o * Db + k0) : zero4();
        }
    }
    float4 bz0 = make_float4(0.f, 0.f, 0.f, 0.f), bz1 = bz0;
    if (cv) {
        const float* bias = (g ? b_a : b_x) + (size_t)blk * Db + c0;
        bz0 = *reinterpret_cast<const float4*>(bias);
        bz1 = *reinterpret_cast<const float4*>(bias + 4);
    }
    uint16_t* const out = (g ? la : lx) + (size_t)blk * Db + c0;

    // Loads are unconditional (no branches, so the wait for a tile does not
    // also wait for the tiles behind it): rows past the range re-read its
    // last row and tiles past the range its last tile.  Such rows only feed
    // tokens whose outputs are not stored.
    struct Regs { v4u v[S]; };
    auto load = [&](Regs& r, int i) {
        const size_t t0 = tr0 + (size_t)min(i, ntile - 1) * TT;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int c = NCH % NT == 0 ? threadIdx.x + s * NT : min((int)threadIdx.x + s * NT, NCH - 1);
            const int row = c / CPR, k8 = (c - row * CPR) * 8;
            r.v[s] = ld16(x + min(t0 + row, tr1 - 1) * D + (size_t)blk * Db + k8);
        }
    };
    auto store = [&](const Regs& r, uint16_t* dst) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int c = threadIdx.x + s * NT;
            const int row = c / CPR, k8 = (c - row * CPR) * 8;
            if (NCH % NT == 0 || c < NCH) st16(dst + row * RS + k8, r.v[s]);
        }
    };
    auto compute = [&](int i, const uint16_t* bufp) {
        if (2 * G::P < NW && !has_unit) return;
        const size_t t0 = tr0 + (size_t)i * TT;
#pragma unroll
        for (int tg = 0; tg < TT / 16; ++tg) {
            const int tok = tg * 16 + col;
            v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                const bool half = G::ODD && ks == G::KS - 1;  // lanes grp >= 2 lie past Db
                const int k0 = 32 * ks + 8 * grp - ((half && grp >= 2) ? 16 : 0);
                v4u xf = ld16(bufp + tok * RS + k0);
                if (half && grp >= 2) xf = zero4();
                a0 = mfma(wf[0][ks], xf, a0);
                a1 = mfma(wf[1][ks], xf, a1);
            }
            const u32x4_t v{pack_bf16x2(a0[0] + bz0.x, a0[1] + bz0.y), pack_bf16x2(a0[2] + bz0.z, a0[3] + bz0.w),
                            pack_bf16x2(a1[0] + bz1.x, a1[1] + bz1.y), pack_bf16x2(a1[2] + bz1.z, a1[3] + bz1.w)};
            if (STAGE) {
                if (cv) *reinterpret_cast<u32x4_t*>(sout + (g * TT + tok) * RS + c0) = v;
            } else if (cv && t0 + tok < tr1) {  // streamed past the caches by default (the better choice for the layer)
                out_store<u32x4_t, LRS_GP_FWD_NT != 0>(out + (t0 + tok) * D, v);
            }
        }
    };
    // the staged logits of tile i, whole rows of Db channels per gate
    constexpr int OCH = 2 * TT * CPR, SO = (OCH + NT - 1) / NT;
    auto flush = [&](int i) {
        const size_t t0 = tr0 + (size_t)i * TT;
#pragma unroll
        for (int s = 0; s < SO; ++s) {
            const int c = threadIdx.x + s * NT;
            if (OCH % NT != 0 && c >= OCH) continue;
            const int gg = c / (TT * CPR), rem = c - gg * TT * CPR, row = rem / CPR, k8 = (rem - row * CPR) * 8;
            if (t0 + row < tr1)
                out_store<u32x4_t, LRS_GP_FWD_NT != 0>((gg ? la : lx) + (t0 + row) * D + (size_t)blk * Db + k8,
                                                       *reinterpret_cast<const u32x4_t*>(sout + (gg * TT + row) * RS + k8));
        }
    };

    // LDS double buffer; tiles i + 1 and i + 2 are in registers or in flight
    // while tile i is multiplied.  The body always runs both halves (a tile
    // past the range stores nothing), so every load is issued on every path
    // and the wait for one tile never covers the tile behind it.
    Regs ra, rb;
    load(ra, 0);
    sched_fence();
    load(rb, 1);
    sched_fence();
    store(ra, buf0);
    load(ra, 2);
    sched_fence();
    __syncthreads();
    for (int i = 0; i < ntile; i += 2) {
        compute(i, buf0);
        sched_fence();
        store(rb, buf1);
        load(rb, i + 3);
        sched_fence();
        __syncthreads();
        if (STAGE) {
            flush(i);
            __syncthreads();  // the staged logits are read before the next tile overwrites them
        }
        compute(i + 1, buf1);
        sched_fence();
        store(ra, buf0);
        load(ra, i + 4);
        sched_fence();
        __syncthreads();
        if (STAGE) {
            flush(i + 1);
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------ dx (adjoint)
// grid (16 blocks, ranges).  dx^T[k][t] = sum_g W_g^T[k][o] dl_g^T[o][t]:
// A = W^T rows (staged transposed through LDS once, then registers), B = dl
// rows (LDS).  Waves per pair: 4 for P = 1, 2 for P = 2..4, 1 for P = 5
// (a workgroup of more than eight waves would cap each at 168 registers);
// the waves of a pair split the four token groups of a tile.
template <int MT>
constexpr int dx_waves() {
    return Geo<MT>::P == 1 ? 4 : (2 * Geo<MT>::P <= 8 ? 2 * Geo<MT>::P : Geo<MT>::P);
}

// tiles requested ahead: two where the registers allow it
template <int MT, bool F32>
constexpr int prefetch_depth() {
    return (F32 || MT >= 9) ? 1 : 2;
}
// tokens per tile of the adjoint kernels: halved for FP32 cotangents of the
// widest blocks, whose staging registers would otherwise spill
template <int MT, bool F32>
constexpr int adj_tile() {
    return (F32 && MT >= 9) ? 32 : TT;
}

// dx_in rows staged through LDS with the cotangent tiles and dx_out written
// back from there as whole token rows (rather than 64-byte pieces per lane
// group); measured faster up to 8 tiles per block, slower for the five-wave
// workgroups of the widest blocks
#ifndef LRS_GP_DX_STAGE
#define LRS_GP_DX_STAGE 1
#endif
template <int MT>
constexpr bool dx_stage() {
    return LRS_GP_DX_STAGE != 0 && MT <= 8;
}

template <int MT, bool F32>
constexpr size_t dx_lds_bytes() {
    constexpr int Db = 16 * MT;
    constexpr size_t tile =
        (size_t)(dx_stage<MT>() ? 3 : 2) * adj_tile<MT, F32>() * (Db + (F32 ? FPAD : XPAD)) * (F32 ? 4 : 2);
    constexpr size_t wt = (size_t)Db * (Db + XPAD) * 2;
    return tile > wt ? tile : wt;
}

template <int MT, bool F32>
__global__ __launch_bounds__(64 * dx_waves<MT>()) void gate_proj_dx_kernel(
    int BL, int D, int range, const uint16_t* __restrict__ w_x, const uint16_t* __restrict__ w_a,
    const void* __restrict__ dlx, const void* __restrict__ dla, const void* dx_in, void* dx_out) {
    using G = Geo<MT>;
    constexpr int Db = G::Db, NW = dx_waves<MT>(), NT = 64 * NW, ES = F32 ? 4 : 2;
    constexpr int RS = Db + (F32 ? FPAD : XPAD), RW = Db + XPAD;
    constexpr int T = adj_tile<MT, F32>();         // tokens per tile
    constexpr int WPP = NW / G::P, TGW = (T / 16) / WPP;  // waves per pair, token groups per wave and tile
    static_assert(TGW >= 1, "every wave owns a token group");
    constexpr bool STAGE = dx_stage<MT>();
    constexpr int DX_PLANES = STAGE ? 3 : 2;
    constexpr int CPR = Db * ES / 16, NCH = T * CPR, S = (NCH + NT - 1) / NT;  // 16-byte chunks per plane
    constexpr int PF = prefetch_depth<MT, F32>();
    extern __shared__ uint16_t gp_lds[];
    // [2 gates (+ dx rows when STAGE)][T][RS] x ES bytes
    unsigned char* const tile = reinterpret_cast<unsigned char*>(gp_lds);
    unsigned char* const sio = tile + (size_t)2 * T * RS * ES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
    const int blk = blockIdx.x;
    const size_t tr0 = (size_t)blockIdx.y * range, tr1 = min((size_t)BL, tr0 + range);
    const int ntile = (int)((tr1 - tr0 + T - 1) / T);
    const int p = wave / WPP;
    const int tgb = (wave - p * WPP) * TGW;
    const int c0 = 32 * p + 8 * grp;
    const bool cv = c0 + 8 <= Db;

    // A fragments of both gates: W_g^T row k = pair_chan(p, col, h), columns o
    v4u wf[2][2][G::KS];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
        if (gg) __syncthreads();
        stage_transposed_bf16(gp_lds, RW, (gg ? w_a : w_x) + (size_t)blk * Db * Db, Db, Db, Db, NT);
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = pair_chan(p, col, h);
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                const int o0 = 32 * ks + 8 * grp;
                wf[gg][h][ks] = (k < Db && o0 < Db) ? ld16(gp_lds + k * RW + o0) : zero4();
            }
        }
    }

    // planes: dl^x, dl^a and (STAGE) the dx_in rows
    struct Regs { v4u v[DX_PLANES][S]; };
    // unconditional loads, as in the forward: rows past the range re-read
    // its last row and only feed tokens whose dx is not stored
    auto load = [&](Regs& r, int i) {
        const size_t t0 = tr0 + (size_t)min(i, ntile - 1) * T;
#pragma unroll
        for (int pl = 0; pl < DX_PLANES; ++pl) {
            const unsigned char* src = reinterpret_cast<const unsigned char*>(pl == 0 ? dlx : (pl == 1 ? dla : dx_in));
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int c = NCH % NT == 0 ? threadIdx.x + s * NT : min((int)threadIdx.x + s * NT, NCH - 1);
                const int row = c / CPR, ch = c - row * CPR;
                r.v[pl][s] = ld16(src + (min(t0 + row, tr1 - 1) * D + (size_t)blk * Db) * ES + ch * 16);
            }
        }
    };
    auto store = [&](const Regs& r) {
#pragma unroll
        for (int pl = 0; pl < DX_PLANES; ++pl)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int c = threadIdx.x + s * NT;
                const int row = c / CPR, ch = c - row * CPR;
                if (NCH % NT == 0 || c < NCH) st16(tile + ((size_t)(pl * T + row) * RS) * ES + ch * 16, r.v[pl][s]);
            }
    };
    // dx_in of the tile, requested before the prefetch of later tiles so
    // that waiting for it does not wait for them; a lane that stores nothing
    // reads inside the range and the block
    struct In { v4u v[TGW][F32 ? 2 : 1]; };
    auto load_in = [&](In& d, int i) {
        const size_t t0 = tr0 + (size_t)i * T;
#pragma unroll
        for (int q = 0; q < TGW; ++q) {
            const int tok = (tgb + q) * 16 + col;
            const size_t src = (min(t0 + tok, tr1 - 1) * D + (size_t)blk * Db + min(c0, Db - 8)) * ES;
#pragma unroll
            for (int u = 0; u < (F32 ? 2 : 1); ++u)
                d.v[q][u] = ld16(reinterpret_cast<const unsigned char*>(dx_in) + src + 16 * u);
        }
    };
    auto compute = [&](int i, const In& d) {
        const size_t t0 = tr0 + (size_t)i * T;
#pragma unroll
        for (int q = 0; q < TGW; ++q) {
            const int tok = (tgb + q) * 16 + col;
            const bool tv = cv && t0 + tok < tr1;
            const size_t dst = ((t0 + tok) * D + (size_t)blk * Db + c0) * ES;
            unsigned char* const sdx = sio + ((size_t)tok * RS + min(c0, Db - 8)) * ES;
            v4u in0, in1 = zero4();
            if constexpr (STAGE) {
                in0 = ld16(sdx);
                if (F32) in1 = ld16(sdx + 16);
            } else {
                in0 = d.v[q][0];
                in1 = d.v[q][F32 ? 1 : 0];
            }
            v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks) {
                    const bool half = G::ODD && ks == G::KS - 1;
                    const int o0 = 32 * ks + 8 * grp - ((half && grp >= 2) ? 16 : 0);
                    const unsigned char* src = tile + ((size_t)(gg * T + tok) * RS + o0) * ES;
                    if (F32) {
                        v4u hi, mid, lo;
                        split3(ld16(src), ld16(src + 16), hi, mid, lo);
                        if (half && grp >= 2) hi = mid = lo = zero4();
                        a0 = mfma(wf[gg][0][ks], hi, a0);
                        a1 = mfma(wf[gg][1][ks], hi, a1);
                        a0 = mfma(wf[gg][0][ks], mid, a0);
                        a1 = mfma(wf[gg][1][ks], mid, a1);
                        a0 = mfma(wf[gg][0][ks], lo, a0);
                        a1 = mfma(wf[gg][1][ks], lo, a1);
                    } else {
                        v4u bf = ld16(src);
                        if (half && grp >= 2) bf = zero4();
                        a0 = mfma(wf[gg][0][ks], bf, a0);
                        a1 = mfma(wf[gg][1][ks], bf, a1);
                    }
                }
            }
            v4u r0, r1 = zero4();
            if (F32) {
                r0 = v4u{__float_as_uint(__uint_as_float(in0.x) + a0[0]), __float_as_uint(__uint_as_float(in0.y) + a0[1]),
                         __float_as_uint(__uint_as_float(in0.z) + a0[2]), __float_as_uint(__uint_as_float(in0.w) + a0[3])};
                r1 = v4u{__float_as_uint(__uint_as_float(in1.x) + a1[0]), __float_as_uint(__uint_as_float(in1.y) + a1[1]),
                         __float_as_uint(__uint_as_float(in1.z) + a1[2]), __float_as_uint(__uint_as_float(in1.w) + a1[3])};
            } else {
                r0 = v4u{pack_bf16x2(bf16_lo(in0.x) + a0[0], bf16_hi(in0.x) + a0[1]),
                         pack_bf16x2(bf16_lo(in0.y) + a0[2], bf16_hi(in0.y) + a0[3]),
                         pack_bf16x2(bf16_lo(in0.z) + a1[0], bf16_hi(in0.z) + a1[1]),
                         pack_bf16x2(bf16_lo(in0.w) + a1[2], bf16_hi(in0.w) + a1[3])};
            }
            if (STAGE) {  // back into the staged row, written out whole by flush()
                if (cv) {
                    st16(sdx, r0);
                    if (F32) st16(sdx + 16, r1);
                }
            } else if (tv) {
                unsigned char* o = reinterpret_cast<unsigned char*>(dx_out) + dst;
                out_store<u32x4_t>(o, u32x4_t{r0.x, r0.y, r0.z, r0.w});
                if (F32) out_store<u32x4_t>(o + 16, u32x4_t{r1.x, r1.y, r1.z, r1.w});
            }
        }
    };
    // the staged dx rows of tile i
    constexpr int OCH = NCH, SO = S;
    auto flush = [&](int i) {
        const size_t t0 = tr0 + (size_t)i * T;
#pragma unroll
        for (int s = 0; s < SO; ++s) {
            const int c = threadIdx.x + s * NT;
            if (OCH % NT != 0 && c >= OCH) continue;
            const int row = c / CPR, ch = c - row * CPR;
            if (t0 + row < tr1) {
                const v4u v = ld16(sio + (size_t)row * RS * ES + ch * 16);
                out_store<u32x4_t>(reinterpret_cast<unsigned char*>(dx_out) + ((t0 + row) * D + (size_t)blk * Db) * ES +
                                       ch * 16,
                                   u32x4_t{v.x, v.y, v.z, v.w});
            }
        }
    };

    // one LDS tile; the next PF tiles in registers or in flight.  Every
    // iteration runs all PF stages (a tile past the range stores nothing),
    // so each load is issued on every path.
    Regs rr[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        load(rr[j], j);
        sched_fence();
    }
    for (int i = 0; i < ntile; i += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            In d;
            if constexpr (!STAGE) load_in(d, i + j);
            sched_fence();
            __syncthreads();  // the previous tile (or the weight staging) is no longer read
            sched_fence();
            store(rr[j]);
            load(rr[j], i + j + PF);
            sched_fence();
            __syncthreads();
            compute(i + j, d);
            if (STAGE) {
                __syncthreads();  // the tile's dx rows are complete
                flush(i + j);
            }
        }
    }
}

// ------------------------------------------------------- dW, db (adjoint)
// grid (16 blocks, ranges of LRS_GP_DW_RANGE tokens).  Partial sums over the
// range: dW[o][k] = sum_t dl^T[o][t] x[t][k] with the tokens as the
// reduction index.  Tiles sit in LDS in their natural layout (rows = tokens)
// and fragments come from transposing LDS reads (ds_read_b64_tr_b16: within
// each 16-lane group, lane i receives element i%4 of the 8 bytes read by
// lanes 4j + i/4, j = 0..3; a lane that reads row t0 + s/4 at channel
// c0 + 4 (s%4) thus hands lane i channel c0 + i at tokens t0..t0+3).  Wave w
// owns R rows (gate, 16-row tile mo) with all MT column tiles plus one bias
// tile whose B operand is the constant column (1, 0, ..., 0): its first
// column is db = sum_t dl, summed by the matrix cores alongside dW.  FP32
// cotangents are split into three BF16 planes when they are staged.
template <int MT>
constexpr int dw_waves() {
    return MT >= 4 ? MT : 4;
}
template <int MT>
constexpr int dw_rows() {
    return (2 * MT + dw_waves<MT>() - 1) / dw_waves<MT>();
}
// LDS row stride (BF16 elements): an odd multiple of 16, so the four rows
// one 16-lane group reads fall on disjoint banks
template <int MT>
constexpr int dw_row() {
    return 16 * (MT | 1);
}
template <int MT, bool F32>
constexpr size_t dw_lds_bytes() {
    return (size_t)adj_tile<MT, F32>() * dw_row<MT>() * 2 * (1 + 2 * (F32 ? 3 : 1));
}

typedef short v4s __attribute__((ext_vector_type(4)));
// eight consecutive tokens (rows p and p + 4 RS.. as two transposing reads) of one channel per lane
__device__ __forceinline__ v4u tr_frag(const uint16_t* p, int rs) {
    typedef __attribute__((address_space(3))) v4s* lp;
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(p + 4 * rs));
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return v4u{ua.x, ua.y, ub.x, ub.y};
}

// four FP32 values -> BF16 hi, mid, lo (exact split, as split3)
__device__ __forceinline__ void split3x4(v4u f, uint2& hi, uint2& mid, uint2& lo) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = f[j] & 0xffff0000u;
        const float r1 = __uint_as_float(f[j]) - __uint_as_float(h[j]);
        m[j] = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(m[j]);
        l[j] = __float_as_uint(r2) & 0xffff0000u;
    }
    hi = make_uint2((h[0] >> 16) | h[1], (h[2] >> 16) | h[3]);
    mid = make_uint2((m[0] >> 16) | m[1], (m[2] >> 16) | m[3]);
    lo = make_uint2((l[0] >> 16) | l[1], (l[2] >> 16) | l[3]);
}

template <int MT, bool F32>
__global__ __launch_bounds__(64 * dw_waves<MT>()) void gate_proj_dw_kernel(
    int BL, int D, int range, const uint16_t* __restrict__ x, const void* __restrict__ dlx,
    const void* __restrict__ dla, float* __restrict__ dw_part, float* __restrict__ db_part) {
    constexpr int Db = 16 * MT, NW = dw_waves<MT>(), NT = 64 * NW, R = dw_rows<MT>();
    constexpr int RS = dw_row<MT>(), ES = F32 ? 4 : 2, NPL = F32 ? 3 : 1;
    constexpr int PF = prefetch_depth<MT, F32>();
    constexpr int T = adj_tile<MT, F32>();  // tokens per tile
    constexpr int XCR = Db / 8, XC = T * XCR;             // 16-byte chunks of x: per row, per tile
    constexpr int LCR = Db * ES / 16, LC = T * LCR;       // of one cotangent tile
    constexpr int SX = (XC + NT - 1) / NT, SL = (LC + NT - 1) / NT;
    extern __shared__ uint16_t gp_lds[];  // x [T][RS], dl [2 gates][NPL planes][T][RS]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
    const int blk = blockIdx.x, r = blockIdx.y;
    const size_t tr0 = (size_t)r * range, tr1 = min((size_t)BL, tr0 + range);
    const int ntile = (int)((tr1 - tr0 + T - 1) / T);

    v4f acc[R][MT + 1];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int n = 0; n <= MT; ++n) acc[j][n] = v4f{0.f, 0.f, 0.f, 0.f};

    // Loads are unconditional (rows past the range re-read its last row,
    // tiles past it its last tile); a row mask, applied when the chunk is
    // written to LDS, zeroes the rows that do not belong to this tile.
    struct Regs {
        v4u x[SX];
        v4u l[2][SL];
        uint32_t okx, okl;  // bit s (+ SL for gate 1): the chunk's token row is in the range
    };
    auto chunk = [&](int s, int nchunks) {
        const int c = threadIdx.x + s * NT;
        return nchunks % NT == 0 ? c : min(c, nchunks - 1);
    };
    auto load = [&](Regs& b, int i) {
        const size_t t0 = tr0 + (size_t)min(i, ntile - 1) * T;
        b.okx = b.okl = 0;
#pragma unroll
        for (int s = 0; s < SX; ++s) {
            const int c = chunk(s, XC), row = c / XCR, c8 = c - row * XCR;
            const size_t t = t0 + row;
            b.okx |= (i < ntile && t < tr1) ? 1u << s : 0u;
            b.x[s] = ld16(x + min(t, tr1 - 1) * D + (size_t)blk * Db + 8 * c8);
        }
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                const int c = chunk(s, LC), row = c / LCR, ch = c - row * LCR;
                const size_t t = t0 + row;
                b.okl |= (i < ntile && t < tr1) ? 1u << (gg * SL + s) : 0u;
                b.l[gg][s] = ld16(reinterpret_cast<const unsigned char*>(gg ? dla : dlx) +
                                  (min(t, tr1 - 1) * D + (size_t)blk * Db) * ES + 16 * ch);
            }
    };
    auto store = [&](const Regs& b, uint16_t* sx) {
        uint16_t* const sl = sx + T * RS;
#pragma unroll
        for (int s = 0; s < SX; ++s) {
            const int c = threadIdx.x + s * NT;
            if (XC % NT != 0 && c >= XC) continue;
            const int row = c / XCR, c8 = c - row * XCR;
            st16(sx + row * RS + 8 * c8, (b.okx >> s & 1u) ? b.x[s] : zero4());
        }
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                const int c = threadIdx.x + s * NT;
                if (LC % NT != 0 && c >= LC) continue;
                const int row = c / LCR, ch = c - row * LCR;
                const v4u v = (b.okl >> (gg * SL + s) & 1u) ? b.l[gg][s] : zero4();
                if (F32) {
                    uint2 hi, mid, lo;
                    split3x4(v, hi, mid, lo);
                    uint16_t* d = sl + ((gg * 3) * T + row) * RS + 4 * ch;
                    *reinterpret_cast<uint2*>(d) = hi;
                    *reinterpret_cast<uint2*>(d + T * RS) = mid;
                    *reinterpret_cast<uint2*>(d + 2 * T * RS) = lo;
                } else {
                    st16(sl + (gg * T + row) * RS + 8 * ch, v);
                }
            }
    };
    const v4u ones = col == 0 ? v4u{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u} : zero4();
    auto compute = [&](const uint16_t* sx) {
        const uint16_t* const sl = sx + T * RS;
#pragma unroll
        for (int kt = 0; kt < T; kt += 32) {
            const int toff = (kt + 8 * grp + (col >> 2)) * RS + 4 * (col & 3);  // this lane's read address
            v4u af[R][NPL];
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int row = wave * R + j;  // gate row / MT, tile row % MT
                const int rc = row < 2 * MT ? row : 0;
                const int gg = rc / MT, mo = rc - gg * MT;
#pragma unroll
                for (int p = 0; p < NPL; ++p) af[j][p] = tr_frag(sl + (gg * NPL + p) * T * RS + toff + mo * 16, RS);
            }
#pragma unroll
            for (int n = 0; n <= MT; ++n) {
                const v4u bf = n < MT ? tr_frag(sx + toff + n * 16, RS) : ones;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    if (2 * MT % NW != 0 && wave * R + j >= 2 * MT) continue;
#pragma unroll
                    for (int p = 0; p < NPL; ++p) acc[j][n] = mfma(af[j][p], bf, acc[j][n]);
                }
            }
        }
    };

    // all PF stages every iteration: a tile past the range is masked to zero
    Regs rr[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        load(rr[j], j);
        sched_fence();
    }
    for (int i = 0; i < ntile; i += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            __syncthreads();
            sched_fence();
            store(rr[j], gp_lds);
            load(rr[j], i + j + PF);
            sched_fence();
            __syncthreads();
            compute(gp_lds);
        }
    }

    // D[o][k]: lane holds o = mo 16 + 4 grp + e, k = n 16 + col
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int row = wave * R + j;
        if (row >= 2 * MT) continue;
        const int gg = row / MT, mo = row - gg * MT;
        float* dst = dw_part + ((((size_t)r * 2 + gg) * 16 + blk) * Db + mo * 16 + 4 * grp) * Db + col;
#pragma unroll
        for (int n = 0; n < MT; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(size_t)e * Db + n * 16] = acc[j][n][e];
        if (col == 0) {
            float* db = db_part + ((size_t)r * 2 + gg) * D + (size_t)blk * Db + mo * 16 + 4 * grp;
            *reinterpret_cast<float4*>(db) = make_float4(acc[j][MT][0], acc[j][MT][1], acc[j][MT][2], acc[j][MT][3]);
        }
    }
}

// ------------------------------------------- adjoint in one pass (BF16)
// grid (16 blocks, ranges of LRS_GP_DW_RANGE tokens).  dx and dW need the
// same cotangent tiles, so one workgroup streams x, dl^x, dl^a and dx_in
// through LDS once and splits its waves by product: waves [0, NWX) form
// dx (the dx kernel's layout: W_g^T fragments in registers, cotangent rows
// as B), waves [NWX, NWX + NWW) form the dW and db partials of the range
// (the dW kernel's layout: transposing LDS reads, accumulators in
// registers).  The two roles run separate copies of one tile loop, so the W
// fragments of one and the accumulators of the other never hold registers
// at the same time; both copies pass the same barriers in the same order.
// The x plane keeps the dW kernel's LDS row stride and the cotangent and dx
// planes the dx kernel's, so each product's reads stay free of bank
// conflicts.  Rows past the range read as zero (range-checked buffer
// loads), which dW needs and dx never stores.  The LDS holds two tiles:
// tile i + 1 is written while tile i is multiplied, so that write needs no
// barrier of its own.  Measured at B=1, L=32768, D=2048: 145 us against
// 101 + 93 us for the dx and dW kernels.  Two tiles in flight (the dx waves
// requesting every tile), the separate row strides and 1024- or 4096-token
// ranges each left it within a microsecond or made it slower.
template <int MT>
constexpr int adj_waves() {
    return dx_waves<MT>() + dw_waves<MT>();
}
// the matrix-core adjoint in one pass: BF16 cotangents and up to 8 tiles per
// block (wider blocks would not fit both roles' registers at four waves per
// SIMD)
template <int MT>
constexpr bool adj_fused() {
    return MT <= 8 && adj_waves<MT>() <= 16;
}
#ifndef LRS_GP_ADJ_DBUF
#define LRS_GP_ADJ_DBUF 1       // two LDS tiles (the next tile is written during the products)
#endif
#ifndef LRS_GP_ADJ_DIRECT
#define LRS_GP_ADJ_DIRECT 0     // dx written by the lanes that form it (measured slower than staged rows)
#endif
template <int MT>
constexpr size_t adj_lds_bytes() {
    constexpr int Db = 16 * MT;
    constexpr size_t tiles = (size_t)(LRS_GP_ADJ_DBUF ? 2 : 1) * TT * (dw_row<MT>() + 3 * (Db + XPAD)) * 2;
    constexpr size_t wts = (size_t)2 * Db * (Db + XPAD) * 2;                                 // W_x^T, W_a^T
    return tiles > wts ? tiles : wts;
}

template <int MT>
__global__ __launch_bounds__(64 * adj_waves<MT>()) void gate_proj_adj_kernel(
    int BL, int D, int range, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_x,
    const uint16_t* __restrict__ w_a, const uint16_t* __restrict__ dlx, const uint16_t* __restrict__ dla,
    const uint16_t* dx_in, uint16_t* dx_out, float* __restrict__ dw_part, float* __restrict__ db_part) {
    using G = Geo<MT>;
    constexpr int Db = G::Db, NWX = dx_waves<MT>(), NWW = dw_waves<MT>(), NT = 64 * (NWX + NWW);
    // row strides: x as in the dW kernel (rows on disjoint banks for the
    // transposing reads), the cotangent and dx planes as in the dx kernel
    // (sixteen consecutive rows on disjoint banks for the 16-byte row reads)
    constexpr int T = TT, RX = dw_row<MT>(), RL = Db + XPAD, RW = Db + XPAD, R = dw_rows<MT>();
    constexpr int WPP = NWX / G::P, TGW = (T / 16) / WPP;  // dx: waves per pair, token groups per wave
    constexpr int CPR = Db / 8, NCH = T * CPR, S = (NCH + NT - 1) / NT;  // 16-byte chunks per plane
    constexpr bool DBUF = LRS_GP_ADJ_DBUF != 0, DIRECT = LRS_GP_ADJ_DIRECT != 0;
    constexpr int TILE = T * (RX + 3 * RL);  // elements of one tile's four planes
    constexpr int PL1 = T * RX, PL3 = T * (RX + 2 * RL);  // plane offsets: dl^x (dl^a follows), dx rows
    static_assert(TGW >= 1 && 64 * (NWX + NWW) <= 1024, "adjoint workgroup shape");
    extern __shared__ uint16_t gp_lds[];  // per tile: x [T][RX], dl^x, dl^a [2][T][RL], dx rows [T][RL]
    const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = blockIdx.x, r = blockIdx.y;
    const size_t tr0 = (size_t)r * range, tr1 = min((size_t)BL, tr0 + range);
    const int ntile = (int)((tr1 - tr0 + T - 1) / T);

    // Tile loads, shared by both roles, through one buffer descriptor per
    // plane whose range is the workgroup's token rows: a row past the range
    // (a ragged last tile, the tiles the pipeline requests past the end)
    // reads as zero and costs no memory access -- the zero rows dW needs and
    // dx never stores.  The offset of a 16-byte chunk is a 32-bit lane value.
    struct Regs {
        v4u v[4][S];  // x, dl^x, dl^a, dx_in
    };
    const int rbytes = (int)((tr1 - tr0) * D * 2);  // at most range * 2560 * 2 bytes
    const char* const src[4] = {reinterpret_cast<const char*>(x), reinterpret_cast<const char*>(dlx),
                                reinterpret_cast<const char*>(dla), reinterpret_cast<const char*>(dx_in)};
    __amdgpu_buffer_rsrc_t rsrc[4];
#pragma unroll
    for (int pl = 0; pl < 4; ++pl)
        rsrc[pl] = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src[pl] + tr0 * D * 2), (short)0, rbytes,
                                                     0x00020000);
    // every word is read once, by the step's last reader of it: cache policy
    // 2 (non-temporal) keeps the planes out of the memory-side cache
    auto load = [&](Regs& b, int i) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int c = NCH % NT == 0 ? threadIdx.x + s * NT : min((int)threadIdx.x + s * NT, NCH - 1);
            const int row = c / CPR, ch = c - row * CPR;
            const uint32_t off = (uint32_t)(((i * T + row) * D + blk * Db + 8 * ch) * 2);
#pragma unroll
            for (int pl = 0; pl < 4; ++pl) b.v[pl][s] = __builtin_amdgcn_raw_buffer_load_b128(rsrc[pl], off, 0, 2);
        }
    };
    // W_x^T and W_a^T of the block, for the dx waves' fragments
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
        stage_transposed_bf16(gp_lds + gg * Db * RW, RW, (gg ? w_a : w_x) + (size_t)blk * Db * Db, Db, Db, Db, NT);
    __syncthreads();

    auto tile_of = [&](int i) { return gp_lds + (DBUF ? (i & 1) * TILE : 0); };
    auto store = [&](const Regs& b, uint16_t* tl) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int c = threadIdx.x + s * NT;
            if (NCH % NT != 0 && c >= NCH) continue;
            const int row = c / CPR, ch = c - row * CPR;
#pragma unroll
            for (int pl = 0; pl < 4; ++pl) st16(tl + (pl ? PL1 + ((pl - 1) * T + row) * RL : row * RX) + 8 * ch, b.v[pl][s]);
        }
    };
    // the staged dx rows of tile i, written out whole (when not DIRECT)
    auto flush = [&](int i, const uint16_t* tl) {
        const size_t t0 = tr0 + (size_t)i * T;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int c = threadIdx.x + s * NT;
            if (NCH % NT != 0 && c >= NCH) continue;
            const int row = c / CPR, ch = c - row * CPR;
            if (t0 + row < tr1)
                out_store<u32x4_t>(reinterpret_cast<char*>(dx_out) + t0 * D * 2 +
                                       (uint32_t)((row * D + blk * Db + 8 * ch) * 2),
                                   __builtin_bit_cast(u32x4_t, ld16(tl + PL3 + row * RL + 8 * ch)));
        }
    };
    // The tile loop of both roles.  With DBUF, tile i + 1 goes to the other
    // LDS tile while tile i is multiplied (that tile was last read before the
    // previous barrier); otherwise a barrier keeps them apart.
    auto run = [&](auto&& compute) {
        Regs rr;
        load(rr, 0);
        sched_fence();
        __syncthreads();  // every dx wave holds its fragments: the tiles may overwrite the weights
        if (DBUF) {
            store(rr, tile_of(0));
            load(rr, 1);
            sched_fence();
            __syncthreads();
        }
        for (int i = 0; i < ntile; ++i) {
            if (DBUF) {
                store(rr, tile_of(i + 1));
                load(rr, i + 2);
            } else {
                store(rr, tile_of(i));
                load(rr, i + 1);
                sched_fence();
                __syncthreads();
            }
            sched_fence();
            compute(i, tile_of(i));
            sched_fence();
            __syncthreads();
            if (!DIRECT) {
                flush(i, tile_of(i));
                __syncthreads();  // the rows are read before a later tile overwrites them
            }
        }
    };

    if (wave < NWX) {
        // ---- dx: A = W_g^T rows (registers), B = cotangent rows
        const int p = wave / WPP, tgb = (wave - p * WPP) * TGW;
        const int c0 = 32 * p + 8 * grp;
        const bool cv = c0 + 8 <= Db;
        v4u wf[2][2][G::KS];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = pair_chan(p, col, h);
#pragma unroll
                for (int ks = 0; ks < G::KS; ++ks) {
                    const int o0 = 32 * ks + 8 * grp;
                    wf[gg][h][ks] = (k < Db && o0 < Db) ? ld16(gp_lds + (gg * Db + k) * RW + o0) : zero4();
                }
            }
        run([&](int i, uint16_t* tl) {
            const uint16_t* const sl = tl + PL1;
            uint16_t* const sio = tl + PL3;
            const size_t t0 = tr0 + (size_t)i * T;
#pragma unroll
            for (int q = 0; q < TGW; ++q) {
                const int tok = (tgb + q) * 16 + col;
                uint16_t* const sdx = sio + tok * RL + min(c0, Db - 8);
                const v4u in0 = ld16(sdx);
                v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
                for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                    for (int ks = 0; ks < G::KS; ++ks) {
                        const bool half = G::ODD && ks == G::KS - 1;
                        const int o0 = 32 * ks + 8 * grp - ((half && grp >= 2) ? 16 : 0);
                        v4u bf = ld16(sl + (gg * T + tok) * RL + o0);
                        if (half && grp >= 2) bf = zero4();
                        a0 = mfma(wf[gg][0][ks], bf, a0);
                        a1 = mfma(wf[gg][1][ks], bf, a1);
                    }
                const v4u r0{pack_bf16x2(bf16_lo(in0.x) + a0[0], bf16_hi(in0.x) + a0[1]),
                             pack_bf16x2(bf16_lo(in0.y) + a0[2], bf16_hi(in0.y) + a0[3]),
                             pack_bf16x2(bf16_lo(in0.z) + a1[0], bf16_hi(in0.z) + a1[1]),
                             pack_bf16x2(bf16_lo(in0.w) + a1[2], bf16_hi(in0.w) + a1[3])};
                if (DIRECT) {
                    if (cv && t0 + tok < tr1)
                        out_store<u32x4_t>(reinterpret_cast<char*>(dx_out) + t0 * D * 2 +
                                               (uint32_t)((tok * D + blk * Db + c0) * 2),
                                           __builtin_bit_cast(u32x4_t, r0));
                } else if (cv) {
                    st16(sdx, r0);
                }
            }
        });
    } else {
        // ---- dW, db: partial sums over the range, tokens as the reduction index
        const int dv = wave - NWX;
        v4f acc[R][MT + 1];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int n = 0; n <= MT; ++n) acc[j][n] = v4f{0.f, 0.f, 0.f, 0.f};
        run([&](int, uint16_t* tl) {
            const uint16_t* const sx = tl;
            const uint16_t* const sl = tl + PL1;
#pragma unroll
            for (int kt = 0; kt < T; kt += 32) {
                const int trow = kt + 8 * grp + (col >> 2);  // this lane's read addresses
                const int tx = trow * RX + 4 * (col & 3), tlo = trow * RL + 4 * (col & 3);
                v4u af[R];
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int row = dv * R + j;  // gate row / MT, tile row % MT
                    const int rc = row < 2 * MT ? row : 0;
                    const int gg = rc / MT, mo = rc - gg * MT;
                    af[j] = tr_frag(sl + gg * T * RL + tlo + mo * 16, RL);
                }
                // one B fragment at a time (the accumulators leave no room
                // to request them all at once)
#pragma unroll
                for (int n = 0; n <= MT; ++n) {
                    const uint32_t one = col == 0 ? 0x3f803f80u : 0u;  // the bias tile's column (1, 0, ..., 0)
                    const v4u bf = n < MT ? tr_frag(sx + tx + n * 16, RX) : v4u{one, one, one, one};
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        if (2 * MT % NWW != 0 && dv * R + j >= 2 * MT) continue;
                        acc[j][n] = mfma(af[j], bf, acc[j][n]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        });
        // D[o][k]: lane holds o = mo 16 + 4 grp + e, k = n 16 + col
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = dv * R + j;
            if (row >= 2 * MT) continue;
            const int gg = row / MT, mo = row - gg * MT;
            float* dst = dw_part + ((((size_t)r * 2 + gg) * 16 + blk) * Db + mo * 16 + 4 * grp) * Db + col;
#pragma unroll
            for (int n = 0; n < MT; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(size_t)e * Db + n * 16] = acc[j][n][e];
            if (col == 0) {
                float* db = db_part + ((size_t)r * 2 + gg) * D + (size_t)blk * Db + mo * 16 + 4 * grp;
                *reinterpret_cast<float4*>(db) =
                    make_float4(acc[j][MT][0], acc[j][MT][1], acc[j][MT][2], acc[j][MT][3]);
            }
        }
    }
}

// Sum of the range partials in range order (FP64): dw [2][16][Db][Db], db [2][D].
// The loads of eight ranges are issued ahead of their additions.
__global__ __launch_bounds__(256) void gate_proj_reduce_kernel(int n_ranges, int nw, int D,
                                                               const float* __restrict__ dw_part,
                                                               const float* __restrict__ db_part,
                                                               float* __restrict__ dw_x, float* __restrict__ dw_a,
                                                               float* __restrict__ db_x, float* __restrict__ db_a) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int half = nw / 2;
    if (e < nw) {
        double s = 0.0;
#pragma unroll 8
        for (int r = 0; r < n_ranges; ++r) s += dw_part[(size_t)r * nw + e];
        if (e < half) dw_x[e] = (float)s;
        else dw_a[e - half] = (float)s;
    } else if (e < nw + 2 * D) {
        const int f = e - nw;
        double s = 0.0;
#pragma unroll 8
        for (int r = 0; r < n_ranges; ++r) s += db_part[(size_t)r * 2 * D + f];
        if (f < D) db_x[f] = (float)s;
        else db_a[f - D] = (float)s;
    }
}

template <class F>
hipError_t allow_lds(F* kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

}  // namespace

int gate_proj_ranges(int BL) { return (int)std::max<int64_t>(1, ceil_div(BL, LRS_GP_DW_RANGE)); }

namespace {

template <int MT>
hipError_t fwd_mt(int BL, int D, const void* x, const void* w_x, const float* b_x, const void* w_a,
                  const float* b_a, void* lx, void* la, hipStream_t s) {
    constexpr int Db = 16 * MT;
    const size_t lds = (size_t)(LRS_GP_FWD_STAGE ? 4 : 2) * TT * (Db + XPAD) * 2;
    const hipError_t e = allow_lds(gate_proj_fwd_kernel<MT>, lds);
    if (e != hipSuccess) return e;
    const int range = stream_range(BL);
    LRS_LAUNCH(K_GATE_PROJ, gate_proj_fwd_kernel<MT>, dim3(16, (unsigned)ceil_div(BL, range)),
               dim3(64 * fwd_waves<MT>()), lds, s, BL, D, range, (const uint16_t*)x, (const uint16_t*)w_x, b_x,
               (const uint16_t*)w_a, b_a, (uint16_t*)lx, (uint16_t*)la);
    return hipGetLastError();
}

template <int MT, bool F32>
hipError_t bwd_mt(int BL, int D, const void* x, const void* w_x, const void* w_a, const void* dlx, const void* dla,
                  const void* dx_in, void* dx_out, float* dw_part, float* db_part, hipStream_t s) {
    constexpr size_t lds_dx = dx_lds_bytes<MT, F32>(), lds_dw = dw_lds_bytes<MT, F32>();
    hipError_t e;
    if constexpr (!F32 && LRS_GP_ADJ_FUSED && adj_fused<MT>()) {
        constexpr size_t lds = adj_lds_bytes<MT>();
        if ((e = allow_lds(gate_proj_adj_kernel<MT>, lds)) != hipSuccess) return e;
        LRS_LAUNCH(K_GATE_PROJ_ADJ, gate_proj_adj_kernel<MT>, dim3(16, (unsigned)gate_proj_ranges(BL)),
                   dim3(64 * adj_waves<MT>()), lds, s, BL, D, LRS_GP_DW_RANGE, (const uint16_t*)x,
                   (const uint16_t*)w_x, (const uint16_t*)w_a, (const uint16_t*)dlx, (const uint16_t*)dla,
                   (const uint16_t*)dx_in, (uint16_t*)dx_out, dw_part, db_part);
        return hipGetLastError();
    }
    if ((e = allow_lds(gate_proj_dx_kernel<MT, F32>, lds_dx)) != hipSuccess) return e;
    if ((e = allow_lds(gate_proj_dw_kernel<MT, F32>, lds_dw)) != hipSuccess) return e;
    const int range = stream_range(BL);
    LRS_LAUNCH(K_GATE_PROJ_DX, (gate_proj_dx_kernel<MT, F32>), dim3(16, (unsigned)ceil_div(BL, range)),
               dim3(64 * dx_waves<MT>()), lds_dx, s, BL, D, range, (const uint16_t*)w_x, (const uint16_t*)w_a, dlx,
               dla, dx_in, dx_out);
    LRS_LAUNCH(K_GATE_PROJ_DW, (gate_proj_dw_kernel<MT, F32>), dim3(16, (unsigned)gate_proj_ranges(BL)),
               dim3(64 * dw_waves<MT>()), lds_dw, s, BL, D, LRS_GP_DW_RANGE, (const uint16_t*)x, dlx, dla, dw_part,
               db_part);
    return hipGetLastError();
}

}  // namespace

#define GP_MT_CASES(F) F(1) F(2) F(3) F(4) F(5) F(6) F(7) F(8) F(9) F(10)

hipError_t launch_gate_proj_fwd(int BL, int D, const void* x, const void* w_x, const float* b_x,
                                const void* w_a, const float* b_a, void* lx, void* la, hipStream_t s) {
    switch (D / 256) {
#define GP_FWD_CASE(M) \
    case M: return fwd_mt<M>(BL, D, x, w_x, b_x, w_a, b_a, lx, la, s);
        GP_MT_CASES(GP_FWD_CASE)
#undef GP_FWD_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gate_proj_bwd(int BL, int D, const void* x, const void* w_x, const void* w_a, const void* dlx,
                                const void* dla, int f32, const void* dx_in, void* dx_out, float* dw_x,
                                float* db_x, float* dw_a, float* db_a, float* dw_part, float* db_part,
                                hipStream_t s) {
    hipError_t e = hipErrorInvalidValue;
    switch (D / 256) {
#define GP_BWD_CASE(M)                                                                                       \
    case M:                                                                                                  \
        e = f32 ? bwd_mt<M, true>(BL, D, x, w_x, w_a, dlx, dla, dx_in, dx_out, dw_part, db_part, s)          \
                : bwd_mt<M, false>(BL, D, x, w_x, w_a, dlx, dla, dx_in, dx_out, dw_part, db_part, s);        \
        break;
        GP_MT_CASES(GP_BWD_CASE)
#undef GP_BWD_CASE
        default: break;
    }
    if (e != hipSuccess) return e;
    const int Db = D / 16;
    const int nw = 2 * 16 * Db * Db;
    LRS_LAUNCH(K_GATE_PROJ_REDUCE, gate_proj_reduce_kernel, dim3((unsigned)ceil_div(nw + 2 * D, 256)), dim3(256), 0,
               s, gate_proj_ranges(BL), nw, D, dw_part, db_part, dw_x, dw_a, db_x, db_a);
    return hipGetLastError();
}

}  // namespace lrs
