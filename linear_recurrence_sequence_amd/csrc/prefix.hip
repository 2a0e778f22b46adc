// prefix.hip -- the grouped linear-work prefix over chunk summaries, shared by
// both scans (real and complex) and both directions (forward states, adjoint
// carries).
//
// Page 'SAMU 与 RG-LRU 的 H800 训练性能对比', sections 04 and 05 (the S_c, L_c,
// U_g, O_g, Q_c displays): with S_c the affine summary of chunk c and group g
// covering chunks g0..g1,
//     U_g = S_{g1} o ... o S_{g0},   O_g = U_{g-1} o ... o U_0,
//     Q_c = L_c o O_g with L_c = S_{c-1} o ... o S_{g0},
// where (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2) and the right operand runs
// first.  The state entering chunk c is Q_c(init).  Three kernels:
//   * compose: one thread per (group, element) forms U_g from its chunks
//     (complex summaries arrive compressed: the transition product of each
//     chunk is rebuilt from two per-chunk scalars, see CompressedSummaries);
//   * group scan: a workgroup owns a few elements and all groups; an LDS
//     Hillis-Steele scan (later o earlier at every step, so the order is
//     kept) gives O_g, and O_g(init), the state entering group g, is stored;
//   * expand: one thread per (group, element) walks the group's chunks from
//     that state, applying S_c and storing the state entering every chunk --
//     that walk is L_c applied to O_g(init).
// With a single group (the serial prefix, G >= C) only the walk runs, from
// init itself.
// Adjoint scans visit chunks and groups in reverse order with the same
// operator.  In compose and expand, lanes map to consecutive elements, so
// every row access is contiguous across the wave.
#include "common.hpp"

namespace lrs {
namespace {

template <int E> struct Aff;
template <> struct Aff<1> {
    float a, b;
    static constexpr int F = 2;
    __device__ static Aff ident() { return {1.f, 0.f}; }
    __device__ static Aff load(const float* p, size_t i) {
        const float2 v = reinterpret_cast<const float2*>(p)[i];
        return {v.x, v.y};
    }
    __device__ void store(float* p, size_t i) const { reinterpret_cast<float2*>(p)[i] = make_float2(a, b); }
    // this o first
    __device__ Aff after(const Aff& f) const { return {a * f.a, fmaf(a, f.b, b)}; }
    __device__ void to_lds(float* s) const { s[0] = a; s[1] = b; }
    __device__ static Aff from_lds(const float* s) { return {s[0], s[1]}; }
};
template <> struct Aff<2> {
    cf a, b;
    static constexpr int F = 4;
    __device__ static Aff ident() { return {{1.f, 0.f}, {0.f, 0.f}}; }
    __device__ static Aff load(const float* p, size_t i) {
        const float4 v = reinterpret_cast<const float4*>(p)[i];
        return {{v.x, v.y}, {v.z, v.w}};
    }
    __device__ void store(float* p, size_t i) const {
        reinterpret_cast<float4*>(p)[i] = make_float4(a.re, a.im, b.re, b.im);
    }
    __device__ Aff after(const Aff& f) const { return {cmul(a, f.a), cfma(a, f.b, b)}; }
    __device__ void to_lds(float* s) const { s[0] = a.re; s[1] = a.im; s[2] = b.re; s[3] = b.im; }
    __device__ static Aff from_lds(const float* s) { return {{s[0], s[1]}, {s[2], s[3]}}; }
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
        const float2 x = reinterpret_cast<const float2*>(p)[i];
        return {{x.x, x.y}};
    }
    __device__ void store(float* p, size_t i) const {
        reinterpret_cast<float2*>(p)[i] = make_float2(v.re, v.im);
    }
    __device__ St apply(const Aff<2>& f) const { return {cfma(f.a, v, f.b)}; }
};

__device__ __forceinline__ int chunk_of(int cc, int C, bool reverse) { return reverse ? C - 1 - cc : cc; }

// Chunk summaries stored whole: (A, B) per (batch, chunk, element).
template <int E>
struct FullSummaries {
    const float* summ;
    int C, W;
    __device__ void bind(int) {}
    __device__ Aff<E> operator()(int b, int c, int w) const {
        return Aff<E>::load(summ, ((size_t)b * C + c) * W + w);
    }
};

// Complex chunk summaries stored compressed: B per (batch, chunk, mode) and
// (G_c, cos D_c, sin D_c) per (batch, chunk); the transition product is
//   A_{c,m} = 2^(kappa_m G_c) e^{i n_c theta_m} e^{i D_c}
// with e^{i n theta} from the mode table (n = K, or K_last for the last
// chunk), and its conjugate for the adjoint (REV) scan.
template <bool REV>
struct CompressedSummaries {
    const float* bpart;
    const float4* chunk;
    const float4* mtab;
    int C, W;
    float kappa;
    float4 ph_full, ph_last;
    __device__ void bind(int w) {
        kappa = mtab[MODE_REC * w].x;
        ph_full = mtab[MODE_REC * w + 2];
        ph_last = mtab[MODE_REC * w + 3];
    }
    __device__ Aff<2> operator()(int b, int c, int w) const {
        const float2 bb = reinterpret_cast<const float2*>(bpart)[((size_t)b * C + c) * W + w];
        Aff<2> f;
        f.a = chunk_transition<REV>(kappa, c == C - 1 ? ph_last : ph_full, chunk[(size_t)b * C + c]);
        f.b = {bb.x, bb.y};
        return f;
    }
};

constexpr int CMP_THREADS = 256;

// U_g for every (batch, group, element), groups numbered in processing order.
template <int E, bool REV, class Sum>
__global__ __launch_bounds__(CMP_THREADS) void prefix_compose_kernel(int C, int G, int NG, int W, Sum sm,
                                                                     float* __restrict__ gsum) {
    const int w = blockIdx.x * CMP_THREADS + threadIdx.x;
    const int q = blockIdx.y, b = blockIdx.z;
    if (w >= W) return;
    sm.bind(w);
    const int c0 = q * G;
    const int n = min(G, C - c0);
    Aff<E> acc = Aff<E>::ident();
#pragma unroll 8
    for (int i = 0; i < n; ++i) acc = sm(b, chunk_of(c0 + i, C, REV), w).after(acc);
    acc.store(gsum, ((size_t)b * NG + q) * W + w);
}

constexpr int SCAN_THREADS = 1024;

// Scan over groups (processing order): MT elements per workgroup, NGB = SCAN_THREADS / MT
// group slots per segment, segments chained through a carried state.
template <int E>
__global__ __launch_bounds__(SCAN_THREADS) void prefix_group_scan_kernel(
    int NG, int W, int MT, const float* __restrict__ gsum, const float* __restrict__ init,
    float* __restrict__ gentry) {
    constexpr int F = Aff<E>::F;
    __shared__ float sh[2][SCAN_THREADS * F];
    const int NGB = SCAN_THREADS / MT;
    const int tid = threadIdx.x;
    const int gl = tid / MT, mt = tid - gl * MT;
    const int w = blockIdx.x * MT + mt;
    const int b = blockIdx.y;
    const bool wok = w < W;
    const int wc = wok ? w : W - 1;

    St<E> carry = init ? St<E>::load(init, (size_t)b * W + wc) : St<E>::zero();
    for (int base = 0; base < NG; base += NGB) {
        const int q = base + gl;
        Aff<E> x = (q < NG) ? Aff<E>::load(gsum, ((size_t)b * NG + q) * W + wc) : Aff<E>::ident();
        int buf = 0;
        x.to_lds(&sh[buf][tid * F]);
        __syncthreads();
        for (int d = 1; d < NGB; d <<= 1) {
            if (gl >= d) x = x.after(Aff<E>::from_lds(&sh[buf][(tid - d * MT) * F]));
            buf ^= 1;
            x.to_lds(&sh[buf][tid * F]);
            __syncthreads();
        }
        // exclusive prefix O_g applied to the carried state
        const Aff<E> ex = gl > 0 ? Aff<E>::from_lds(&sh[buf][(tid - MT) * F]) : Aff<E>::ident();
        const Aff<E> last = Aff<E>::from_lds(&sh[buf][((NGB - 1) * MT + mt) * F]);
        if (q < NG && wok) carry.apply(ex).store(gentry, ((size_t)b * NG + q) * W + w);
        carry = carry.apply(last);
        __syncthreads();
    }
}

// State entering every chunk of group q from the state entering the group
// (gentry NULL: the initial state is zero).
template <int E, bool REV, class Sum>
__global__ __launch_bounds__(CMP_THREADS) void prefix_expand_kernel(int C, int G, int NG, int W, Sum sm,
                                                                    const float* __restrict__ gentry,
                                                                    float* __restrict__ entries) {
    const int w = blockIdx.x * CMP_THREADS + threadIdx.x;
    const int q = blockIdx.y, b = blockIdx.z;
    if (w >= W) return;
    sm.bind(w);
    const int c0 = q * G;
    const int n = min(G, C - c0);
    St<E> h = gentry ? St<E>::load(gentry, ((size_t)b * NG + q) * W + w) : St<E>::zero();
#pragma unroll 8
    for (int i = 0; i < n; ++i) {
        const int c = chunk_of(c0 + i, C, REV);
        const Aff<E> sc = sm(b, c, w);
        h.store(entries, ((size_t)b * C + c) * W + w);
        h = h.apply(sc);
    }
}

template <int E, bool REV, class Sum>
void run_prefix(const Chunking& ch, int W, Sum sm, float* gsum, const float* init, float* entries,
                hipStream_t s) {
    const dim3 wgrid((unsigned)ceil_div(W, CMP_THREADS), ch.NG, ch.B);
    if (ch.NG == 1) {
        // a single group (the serial prefix): the walk starts from init itself
        LRS_LAUNCH(K_PREFIX_ENTRIES, (prefix_expand_kernel<E, REV, Sum>), wgrid, dim3(CMP_THREADS), 0, s,
                   ch.C, ch.G, ch.NG, W, sm, init, entries);
        return;
    }
    float* gentry = gsum + (size_t)ch.B * ch.NG * W * 2 * E;
    // group slots per segment: all groups when they fit, with >= 8 elements
    // per workgroup so every group row is read as >= 8 contiguous elements
    int slots = 1;
    while (slots < ch.NG && slots < SCAN_THREADS / 8) slots <<= 1;
    const int MT = SCAN_THREADS / slots;
    const dim3 sgrid((unsigned)ceil_div(W, MT), ch.B);
    LRS_LAUNCH(K_PREFIX_GROUPS, (prefix_compose_kernel<E, REV, Sum>), wgrid, dim3(CMP_THREADS), 0, s, ch.C,
               ch.G, ch.NG, W, sm, gsum);
    LRS_LAUNCH(K_PREFIX_OUTER, (prefix_group_scan_kernel<E>), sgrid, dim3(SCAN_THREADS), 0, s, ch.NG, W, MT,
               (const float*)gsum, init, gentry);
    LRS_LAUNCH(K_PREFIX_ENTRIES, (prefix_expand_kernel<E, REV, Sum>), wgrid, dim3(CMP_THREADS), 0, s, ch.C,
               ch.G, ch.NG, W, sm, (const float*)gentry, entries);
}

}  // namespace


hipError_t launch_prefix(int elem, bool reverse, const Chunking& ch, int W, const PrefixSummaries& sm,
                         float* gsum, const float* init, float* entries, hipStream_t s) {
    if (elem == 2) {
        if (reverse)
            run_prefix<2, true>(ch, W, CompressedSummaries<true>{sm.bpart, (const float4*)sm.chunk,
                                                                 (const float4*)sm.mtab, ch.C, W},
                                gsum, init, entries, s);
        else
            run_prefix<2, false>(ch, W, CompressedSummaries<false>{sm.bpart, (const float4*)sm.chunk,
                                                                   (const float4*)sm.mtab, ch.C, W},
                                 gsum, init, entries, s);
    } else {
        if (reverse) run_prefix<1, true>(ch, W, FullSummaries<1>{sm.full, ch.C, W}, gsum, init, entries, s);
        else run_prefix<1, false>(ch, W, FullSummaries<1>{sm.full, ch.C, W}, gsum, init, entries, s);
    }
    return hipGetLastError();
}

}  // namespace lrs
