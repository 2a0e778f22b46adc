// common.hpp -- device helpers shared by the gfx950 scan kernels.
//
// Storage formats: BF16 tensors travel as packed pairs in 32-bit words (low
// half = element 2k, high half = element 2k+1), complex values as (Re, Im)
// pairs, chunk summaries as affine maps (A, B) with h -> A h + B.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "internal.hpp"

namespace lrs {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---------------------------------------------------------------- BF16 ---
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even of two FP32 values into one packed BF16 pair
// (a single v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------- output streams ---
// Stores of the large [B, L, *] outputs (y, db, dx, ...), which no later
// kernel of the same pass reads.  With LRS_STREAM_NT they carry the
// non-temporal hint, so they do not settle in the memory-side cache as dirty
// lines that a later kernel's reads must first write back.
#ifndef LRS_STREAM_NT
#define LRS_STREAM_NT 1
#endif
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <class T, bool NT = (LRS_STREAM_NT != 0)>
__device__ __forceinline__ void out_store(void* p, T v) {
    if (NT) __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
    else *reinterpret_cast<T*>(p) = v;
}
__device__ __forceinline__ void out_u32(void* p, uint32_t a) { out_store<uint32_t>(p, a); }
__device__ __forceinline__ void out_u32x2(void* p, uint32_t a, uint32_t b) { out_store<u32x2_t>(p, u32x2_t{a, b}); }
__device__ __forceinline__ void out_u32x4(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    out_store<u32x4_t>(p, u32x4_t{a, b, c, d});
}
__device__ __forceinline__ void out_f32x2(void* p, float a, float b) { out_store<f32x2_t>(p, f32x2_t{a, b}); }
__device__ __forceinline__ void out_f32x4(void* p, float a, float b, float c, float d) {
    out_store<f32x4_t>(p, f32x4_t{a, b, c, d});
}

// -------------------------------------------------------------- complex ---
struct cf { float re, im; };

__device__ __forceinline__ cf cmul(cf a, cf b) {
    return {fmaf(a.re, b.re, -a.im * b.im), fmaf(a.re, b.im, a.im * b.re)};
}
// a * b + c
__device__ __forceinline__ cf cfma(cf a, cf b, cf c) {
    return {fmaf(a.re, b.re, fmaf(-a.im, b.im, c.re)), fmaf(a.re, b.im, fmaf(a.im, b.re, c.im))};
}
// conj(a) * b
__device__ __forceinline__ cf cmulc(cf a, cf b) {
    return {fmaf(a.re, b.re, a.im * b.im), fmaf(a.re, b.im, -a.im * b.re)};
}
// conj(a) * b + c
__device__ __forceinline__ cf cfmac(cf a, cf b, cf c) {
    return {fmaf(a.re, b.re, fmaf(a.im, b.im, c.re)), fmaf(a.re, b.im, fmaf(-a.im, b.re, c.im))};
}

// ------------------------------------------------------- mode constants ---
// Per-mode static spectrum.  The unit phasor e^{i theta} is kept as an
// unevaluated sum hi + lo of two FP32 pairs (evaluated in FP64, split once)
// so that its rounding does not act as a fixed per-mode bias repeated at
// every step of a long recurrence.  The controller kernel writes one record
// per mode into the saved forward state; every other kernel reads it.
struct ModeConst {
    float kappa;           // -nu * log2(e): rho_t = 2^(kappa * E_t)
    float ch, sh, cl, sl;  // cos(theta) = ch + cl, sin(theta) = sh + sl
    float nu;
};

__device__ __forceinline__ ModeConst mode_const(float nu, float theta) {
    ModeConst k;
    double c, s;
    sincos((double)theta, &s, &c);
    k.ch = (float)c;
    k.cl = (float)(c - (double)k.ch);
    k.sh = (float)s;
    k.sl = (float)(s - (double)k.sh);
    k.kappa = (float)(-(double)nu * 1.4426950408889634074);
    k.nu = nu;
    return k;
}

// e^{i n theta} for a whole chunk of n tokens, split like the unit phasor
// (hi + lo pairs from an FP64 evaluation).  With it, the product of a chunk's
// transitions has the closed form (page 'SAMU strengthened-baseline H800
// report', 'Candidates that remain disabled', the compressed G/D closure)
//   prod_t lambda_{t,m} = exp(-nu_m G_c) e^{i n theta_m} e^{i D_c},
//   G_c = sum_t E_t, D_c = sum_t d_t.
struct ChunkPhase { float ch, sh, cl, sl; };

__device__ __forceinline__ ChunkPhase chunk_phase(float theta, int n) {
    ChunkPhase p;
    double s, c;
    sincos((double)n * (double)theta, &s, &c);
    p.ch = (float)c;
    p.cl = (float)(c - (double)p.ch);
    p.sh = (float)s;
    p.sl = (float)(s - (double)p.sh);
    return p;
}

// Four float4 per mode: (kappa, ch, sh, cl), (sl, nu, 0, 0), then the chunk
// phasors e^{i K theta} and e^{i K_last theta} as (ch, sh, cl, sl).
constexpr int MODE_REC = 4;

__device__ __forceinline__ void store_mode(float4* tab, int m, const ModeConst& k, const ChunkPhase& full,
                                           const ChunkPhase& last) {
    tab[MODE_REC * m] = make_float4(k.kappa, k.ch, k.sh, k.cl);
    tab[MODE_REC * m + 1] = make_float4(k.sl, k.nu, 0.f, 0.f);
    tab[MODE_REC * m + 2] = make_float4(full.ch, full.sh, full.cl, full.sl);
    tab[MODE_REC * m + 3] = make_float4(last.ch, last.sh, last.cl, last.sl);
}

__device__ __forceinline__ ModeConst load_mode(const float4* __restrict__ tab, int m) {
    const float4 a = tab[MODE_REC * m], b = tab[MODE_REC * m + 1];
    ModeConst k;
    k.kappa = a.x; k.ch = a.y; k.sh = a.z; k.cl = a.w;
    k.sl = b.x; k.nu = b.y;
    return k;
}

// Transition of one mode at one token (page section 05, the lambda display):
//   lambda = exp(-nu E_t) [(cos th C_t - sin th S_t) + i (sin th C_t + cos th S_t)]
// E, C, S are the token's shared special functions.
__device__ __forceinline__ cf mode_lambda(const ModeConst& k, float E, float C, float S) {
    float rho = __builtin_amdgcn_exp2f(k.kappa * E);
    float rr = fmaf(k.ch, C, fmaf(-k.sh, S, k.cl));
    float ri = fmaf(k.sh, C, fmaf(k.ch, S, k.sl));
    return {rho * rr, rho * ri};
}

// Transition product of a whole chunk for one mode, from the chunk's record
// (G_c, cos D_c, sin D_c) and the mode's chunk phasor e^{i n theta} (n = K,
// or K_last for the last chunk) kept as (ch, sh, cl, sl):
//   A = 2^(kappa G_c) e^{i n theta} e^{i D_c};
// the adjoint scan uses its conjugate (REV).
template <bool REV>
__device__ __forceinline__ cf chunk_transition(float kappa, float4 ph, float4 rec) {
    const float re = fmaf(ph.x, rec.y, -ph.y * rec.z) + fmaf(ph.z, rec.y, -ph.w * rec.z);
    const float im = fmaf(ph.x, rec.z, ph.y * rec.y) + fmaf(ph.z, rec.z, ph.w * rec.y);
    const float rho = __builtin_amdgcn_exp2f(kappa * rec.x);
    return {rho * re, REV ? -rho * im : rho * im};
}

// The 32-bit words of one chunk's rows of a [B, L, M] word tensor, read
// through a raw buffer descriptor whose range ends at the chunk's last token:
// a row past it (token i >= kc of a partial last chunk) reads as 0, with no
// branch and no per-load clamp, and no access can leave the chunk.  The
// token offset goes into the per-lane offset, which the range check covers
// (the scalar offset it does not).  0x00020000 is the gfx9 descriptor word 3
// for raw 32-bit loads.
struct ChunkRows {
    __amdgpu_buffer_rsrc_t rsrc;
    int M;
    __device__ ChunkRows(const uint32_t* chunk_row0, int kc, int M_)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(chunk_row0), (short)0, kc * M_ * 4,
                                                 0x00020000)),
          M(M_) {}
    __device__ uint32_t load(int i, int m) const {
        return __builtin_amdgcn_raw_buffer_load_b32(rsrc, (i * M + m) * 4, 0, 0);
    }
    // the same with the non-temporal hint, for words nothing reads again
    __device__ uint32_t load_nt(int i, int m) const {
        return __builtin_amdgcn_raw_buffer_load_b32(rsrc, (i * M + m) * 4, 0, 2);
    }
};

// Stores into one chunk's rows of a [B, L, M] tensor of `eb`-byte elements
// (4: a packed BF16 pair, 8: an FP32 pair) through a raw buffer descriptor:
// the token's row offset goes into the scalar offset and the lane's into the
// vector offset, so a store needs no per-token address arithmetic in vector
// registers.  The stores carry the output streams' cache policy.
struct ChunkOut {
    __amdgpu_buffer_rsrc_t rsrc;
    int stride;  // bytes per token row
    __device__ ChunkOut(void* chunk_row0, int kc, int M, int eb)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(chunk_row0, (short)0, kc * M * eb, 0x00020000)),
          stride(M * eb) {}
    __device__ void u32(int i, uint32_t voff, uint32_t v) const {
        __builtin_amdgcn_raw_buffer_store_b32(v, rsrc, voff, i * stride, LRS_STREAM_NT ? 2 : 0);
    }
    __device__ void f32x2(int i, uint32_t voff, float a, float b) const {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(a), __float_as_uint(b)}, rsrc, voff,
                                              i * stride, LRS_STREAM_NT ? 2 : 0);
    }
};

// Orders LDS traffic among the lanes of one wave (a region no other wave
// touches): the wave's LDS instructions execute in program order, so only
// the compiler has to be kept from moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A wave-uniform value the optimizer cannot see through.  Guarding each token
// step of a serial recurrence with `i < opaque(n)` costs one scalar compare and
// branch, and puts every step in its own basic block, so instruction
// selection cannot hoist all of a chunk's transitions (and their LDS control
// reads) ahead of the chain -- which would cost far more registers than the
// latency it hides.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// A per-lane value the optimizer cannot see through: functions of it are
// computed again instead of being kept live from an earlier evaluation.
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Per-token control record written by the controller kernel: E = e^c,
// (C, S) = (cos d, sin d) and d itself.
struct TokenCtl { float E, C, S, d; };

// Per-chunk record of the compressed summaries: (G_c, cos D_c, sin D_c, 0).
struct ChunkCtl { float G, cD, sD, pad; };


// ------------------------------------------------ group hand-off words ---
// The single-pass scans hand the state between groups of chunks through
// 64-bit words: (1 << 32 | float bits), written and read with relaxed
// device-scope atomics.  The area starts zeroed, so a word is valid exactly
// when its high half is 1; a word is never torn, so a reader that sees every
// word it needs valid holds consistent values, and no fence is needed
// between words.  Per (group, mode) two words: the affine part B of the
// group's map U (a group inside a segment) or the state leaving the group
// (a segment's last group).  The transition part A of U is not published:
// a reader forms it from the chunk records exactly as the group itself does.
constexpr int SCAN_PUB_WORDS = 2;

// Word `i` of a group for one lane: `grp` is the group's (wave-uniform) first
// word, `off` the lane's byte offset (mode * 8) and `Mb` = M * 8, so the
// address is a uniform base plus a 32-bit lane offset.
__device__ __forceinline__ uint64_t* pub_word(const uint64_t* grp, int i, uint32_t Mb, uint32_t off) {
    return reinterpret_cast<uint64_t*>(const_cast<char*>(reinterpret_cast<const char*>(grp)) +
                                       (size_t)i * Mb + off);
}
__device__ __forceinline__ uint64_t pub_load(const uint64_t* grp, int i, uint32_t Mb, uint32_t off) {
    return __hip_atomic_load(pub_word(grp, i, Mb, off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pub_store(uint64_t* grp, int i, uint32_t Mb, uint32_t off, float v) {
    __hip_atomic_store(pub_word(grp, i, Mb, off), (uint64_t(1) << 32) | (uint64_t)__float_as_uint(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool pub_ok(uint64_t w) { return (uint32_t)(w >> 32) == 1u; }
__device__ __forceinline__ float pub_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// The two words of an earlier group for this lane's mode, once both are
// published.
__device__ __forceinline__ float2 wait_pair(const uint64_t* grp, uint32_t Mb, uint32_t off, int polls) {
    float2 v = make_float2(__builtin_nanf(""), __builtin_nanf(""));  // kept if the wait expires
    bool ok = false;
    for (int it = 0; it < polls; ++it) {
        if (!ok) {
            // the lane offset afresh each poll: addresses kept across the
            // loop would cost two registers each
            const uint32_t o = opaque_v(off);
            const uint64_t w0 = pub_load(grp, 0, Mb, o), w1 = pub_load(grp, 1, Mb, o);
            if (pub_ok(w0) && pub_ok(w1)) {
                v = make_float2(pub_val(w0), pub_val(w1));
                ok = true;
            }
        }
        if (__all(ok)) break;
        __builtin_amdgcn_s_sleep(1);
    }
    return v;
}

// Where the chunks of a group come from: chunk records [C] of the row, the
// mode's chunk phasors (e^{i K theta} and, for the last chunk, e^{i K_last
// theta}) and kappa; processing order pc maps to chunk pc (forward) or
// C - 1 - pc (REV, the adjoint).
struct GroupChunks {
    const float4* rec;
    float4 ph_full, ph_last;
    float kappa;
    int C;
};

// The transition part of group j's map U_j for this lane's mode: the product
// of its chunks' transitions in processing order, formed with the same
// operations as the group's own table (chunk_transition, then cmul).
template <bool REV>
__device__ __forceinline__ cf group_transition(const GroupChunks& gc, int G, int j) {
    cf ua = {1.f, 0.f};
    for (int i = 0; i < G; ++i) {
        const int pc = j * G + i;
        const int c = REV ? gc.C - 1 - pc : pc;
        const cf a = chunk_transition<REV>(gc.kappa, c == gc.C - 1 ? gc.ph_last : gc.ph_full, gc.rec[c]);
        ua = cmul(a, ua);
    }
    return ua;
}

// The state entering group q (processing order) of one batch row, for this
// lane's mode `mc`; every wave of the workgroup calls it (it holds two
// workgroup barriers).  comp [G][64]: the (A, B) map of each of the group's
// chunks in processing order (wave w's at w); look [G][64]: scratch.
// seed: the state before the first group ([M] complex, NULL = 0); pub: the
// row's [NG][SCAN_PUB_WORDS][M] words.
//
// Fixed order of evaluation.  The groups form segments of G consecutive
// groups.  The last group of a segment publishes the state leaving it (its
// chunks' maps applied in order to the state entering it); every other group
// publishes the B part of U_q = S_{G-1} o ... o S_0.  Group q takes the state
// leaving the previous segment (the seed for the first) and applies the U of
// the segment's groups before it, oldest first: at most G - 1 maps and one
// state, read by G waves at once.  Which words a group reads and the order it
// applies them in depend only on q and G, never on timing, so the result is
// bitwise the same on every run.  The only serial dependence across
// workgroups is the chain of segment states, one link per G groups.
//
// Progress.  Workgroups are dispatched in grid order (mode tiles fastest,
// then groups), and a workgroup only waits for words of lower-numbered
// groups of its own row and mode tile, which were dispatched before it and
// never wait for it, so every wait ends.  Each wait is nevertheless bounded
// (`polls` polls); a wait that expires yields NaN, which then reaches every
// output downstream of it.
template <bool REV>
__device__ __forceinline__ float4 group_handoff(const float4* comp, float4* look, int G, int w, int lane, int q,
                                                int NG, int M, int mc, bool active, const float2* seed,
                                                uint64_t* pub, const GroupChunks& gc, int polls) {
    constexpr int GL = 64;
    const uint32_t Mb = (uint32_t)M * 8u, moff = (uint32_t)mc * 8u;
    uint64_t* mine = pub + (size_t)q * SCAN_PUB_WORDS * M;  // wave-uniform
    const int nprev = q % G;                          // earlier groups of this segment
    const bool seg_last = nprev == G - 1 || q == NG - 1;
    if (w == 0 && active && q + 1 < NG && !seg_last) {
        // the B part of U_q = S_{G-1} o ... o S_0 (the right operand first),
        // published at once
        cf ub = {0.f, 0.f};
        for (int j = 0; j < G; ++j) {  // all G chunks: a group short of G chunks is the last one
            const float4 f = comp[j * GL + lane];
            ub = cfma({f.x, f.y}, ub, {f.z, f.w});
        }
        pub_store(mine, 0, Mb, moff, ub.re);
        pub_store(mine, 1, Mb, moff, ub.im);
    }
    // wave w < nprev reads U of group q-1-w, wave nprev the state entering
    // the segment
    if (w < nprev) {
        const int j = q - 1 - w;
        const cf ua = group_transition<REV>(gc, G, j);
        const float2 ub = wait_pair(pub + (size_t)j * SCAN_PUB_WORDS * M, Mb, moff, polls);
        look[w * GL + lane] = make_float4(ua.re, ua.im, ub.x, ub.y);
    } else if (w == nprev) {
        float2 zs = make_float2(0.f, 0.f);
        if (q - nprev > 0) zs = wait_pair(pub + (size_t)(q - nprev - 1) * SCAN_PUB_WORDS * M, Mb, moff, polls);
        else if (seed) zs = seed[mc];
        look[w * GL + lane] = make_float4(zs.x, zs.y, 0.f, 0.f);
    }
    __syncthreads();
    if (w == 0) {
        const float4 zs = look[nprev * GL + lane];
        cf z = {zs.x, zs.y};
        for (int v = nprev - 1; v >= 0; --v) {  // oldest first
            const float4 f = look[v * GL + lane];
            z = cfma({f.x, f.y}, z, {f.z, f.w});
        }
        if (active && q + 1 < NG && seg_last) {
            // the state leaving the group, for the next segment: this
            // group's chunks applied in order, as in the chain
            cf zo = z;
            for (int j = 0; j < G; ++j) {
                const float4 f = comp[j * GL + lane];
                zo = cfma({f.x, f.y}, zo, {f.z, f.w});
            }
            pub_store(mine, 0, Mb, moff, zo.re);
            pub_store(mine, 1, Mb, moff, zo.im);
        }
        look[lane] = make_float4(z.re, z.im, 0.f, 0.f);
    }
    __syncthreads();
    return look[lane];
}

// ------------------------------------------------------ wave reductions ---
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace lrs
