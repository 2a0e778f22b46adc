// prefix.hip -- the grouped linear-work prefix over chunk summaries.
//
// Page 'SAMU 与 RG-LRU 的 H800 训练性能对比', sections 04 and 05 (the S_c, L_c,
// U_g, O_g, Q_c displays): with S_c the affine summary of chunk c and group g
// covering chunks g0..g1,
//     U_g = S_{g1} o ... o S_{g0},   O_g = U_{g-1} o ... o U_0,
//     Q_c = L_c o O_g with L_c = S_{c-1} o ... o S_{g0},
// and (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2) -- the right operand runs
// first.  The state entering chunk c is Q_c(init): three kernels compute
// U_g (one thread per group and mode), O_g(init) (one thread per mode, serial
// over groups) and then walk each group applying S_c to produce every entry
// state.  With a single group the first two steps vanish and the walk is the
// serial chunk-to-chunk propagation.  Adjoint scans visit the chunks in
// reverse order with the same operator.
//
// Threads map to modes/channels, so every load and store is coalesced across
// the wave and no cross-lane traffic is needed.
#include "common.hpp"

namespace lrs {
namespace {

template <int E> struct Aff;
template <> struct Aff<1> {
    float a, b;
    __device__ static Aff ident() { return {1.f, 0.f}; }
    __device__ static Aff load(const float* p, size_t i) {
        float2 v = reinterpret_cast<const float2*>(p)[i];
        return {v.x, v.y};
    }
    __device__ void store(float* p, size_t i) const { reinterpret_cast<float2*>(p)[i] = make_float2(a, b); }
    // this o first
    __device__ Aff after(const Aff& f) const { return {a * f.a, fmaf(a, f.b, b)}; }
};
template <> struct Aff<2> {
    cf a, b;
    __device__ static Aff ident() { return {{1.f, 0.f}, {0.f, 0.f}}; }
    __device__ static Aff load(const float* p, size_t i) {
        float4 v = reinterpret_cast<const float4*>(p)[i];
        return {{v.x, v.y}, {v.z, v.w}};
    }
    __device__ void store(float* p, size_t i) const {
        reinterpret_cast<float4*>(p)[i] = make_float4(a.re, a.im, b.re, b.im);
    }
    __device__ Aff after(const Aff& f) const { return {cmul(a, f.a), cfma(a, f.b, b)}; }
};

template <int E> struct St;
template <> struct St<1> {
    float v;
    __device__ static St zero() { return {0.f}; }
    __device__ static St load(const float* p, size_t i) { return {p[i]}; }
    __device__ void store(float* p, size_t i) const { p[i] = v; }
    __device__ St apply(const Aff<1>& f) const { return {fmaf(f.a, v, f.b)}; }
};
template <> struct St<2> {
    cf v;
    __device__ static St zero() { return {{0.f, 0.f}}; }
    __device__ static St load(const float* p, size_t i) {
        float2 x = reinterpret_cast<const float2*>(p)[i];
        return {{x.x, x.y}};
    }
    __device__ void store(float* p, size_t i) const {
        reinterpret_cast<float2*>(p)[i] = make_float2(v.re, v.im);
    }
    __device__ St apply(const Aff<2>& f) const { return {cfma(f.a, v, f.b)}; }
};

constexpr int PFX_THREADS = 256;

__device__ __forceinline__ int chunk_of(int cc, int C, bool reverse) { return reverse ? C - 1 - cc : cc; }

// U_g for every (batch, group, mode).
template <int E, bool REV>
__global__ __launch_bounds__(PFX_THREADS) void prefix_groups_kernel(
    int C, int G, int NG, int W, const float* __restrict__ summ, float* __restrict__ grp) {
    const int w = blockIdx.x * PFX_THREADS + threadIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    if (w >= W) return;
    const int c0 = g * G;
    const int n = min(G, C - c0);
    Aff<E> acc = Aff<E>::ident();
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        const int c = chunk_of(c0 + i, C, REV);
        acc = Aff<E>::load(summ, ((size_t)b * C + c) * W + w).after(acc);
    }
    acc.store(grp, ((size_t)b * NG + g) * W + w);
}

// O_g(init) for every group, serial over the groups of one (batch, mode).
template <int E>
__global__ __launch_bounds__(PFX_THREADS) void prefix_outer_kernel(
    int NG, int W, const float* __restrict__ grp, const float* __restrict__ init,
    float* __restrict__ grp_in) {
    const int w = blockIdx.x * PFX_THREADS + threadIdx.x;
    const int b = blockIdx.y;
    if (w >= W) return;
    St<E> h = init ? St<E>::load(init, (size_t)b * W + w) : St<E>::zero();
#pragma unroll 4
    for (int g = 0; g < NG; ++g) {
        const size_t i = ((size_t)b * NG + g) * W + w;
        h.store(grp_in, i);
        h = h.apply(Aff<E>::load(grp, i));
    }
}

// Entry state of every chunk: start from O_g(init) and apply S_c in order.
template <int E, bool REV>
__global__ __launch_bounds__(PFX_THREADS) void prefix_entries_kernel(
    int C, int G, int NG, int W, const float* __restrict__ summ,
    const float* __restrict__ grp_in, const float* __restrict__ init,
    float* __restrict__ entries) {
    const int w = blockIdx.x * PFX_THREADS + threadIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    if (w >= W) return;
    St<E> h;
    if (NG > 1) h = St<E>::load(grp_in, ((size_t)b * NG + g) * W + w);
    else h = init ? St<E>::load(init, (size_t)b * W + w) : St<E>::zero();
    const int c0 = g * G;
    const int n = min(G, C - c0);
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        const int c = chunk_of(c0 + i, C, REV);
        const size_t idx = ((size_t)b * C + c) * W + w;
        h.store(entries, idx);
        h = h.apply(Aff<E>::load(summ, idx));
    }
}

template <int E, bool REV>
hipError_t prefix_impl(const Chunking& ch, int W, const float* summ, float* grp, float* grp_in,
                       const float* init, float* entries, hipStream_t s) {
    const dim3 blk(PFX_THREADS);
    const int wx = (int)ceil_div(W, PFX_THREADS);
    if (ch.NG > 1) {
        LRS_LAUNCH(K_PREFIX_GROUPS, (prefix_groups_kernel<E, REV>), dim3(wx, ch.NG, ch.B), blk, 0, s,
                   ch.C, ch.G, ch.NG, W, summ, grp);
        LRS_LAUNCH(K_PREFIX_OUTER, (prefix_outer_kernel<E>), dim3(wx, ch.B), blk, 0, s,
                   ch.NG, W, (const float*)grp, init, grp_in);
    }
    LRS_LAUNCH(K_PREFIX_ENTRIES, (prefix_entries_kernel<E, REV>), dim3(wx, ch.NG, ch.B), blk, 0, s,
               ch.C, ch.G, ch.NG, W, summ, (const float*)grp_in, init, entries);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefix(int elem, bool reverse, const Chunking& ch, int W, const float* summ,
                         float* grp, float* grp_in, const float* init, float* entries,
                         hipStream_t s) {
    if (elem == 2)
        return reverse ? prefix_impl<2, true>(ch, W, summ, grp, grp_in, init, entries, s)
                       : prefix_impl<2, false>(ch, W, summ, grp, grp_in, init, entries, s);
    return reverse ? prefix_impl<1, true>(ch, W, summ, grp, grp_in, init, entries, s)
                   : prefix_impl<1, false>(ch, W, summ, grp, grp_in, init, entries, s);
}

}  // namespace lrs
