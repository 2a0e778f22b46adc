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
