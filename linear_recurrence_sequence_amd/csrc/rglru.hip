// rglru.hip -- RG-LRU real gated scan for gfx950, on the same chunked-affine
// primitive as the SAMU scan.
//
// Page 'SAMU 与 RG-LRU 的 H800 训练性能对比', section 04:
//   g^x = sigmoid(l^x), g^a = sigmoid(l^a), a_t = exp(-8 g^a softplus(alpha)),
//   b_t = x_t g^x sqrt(max(1 - a_t^2, 0)), h_t = a_t h_{t-1} + b_t;
//   a segment start sets a_t = 0 and the normalization multiplier to 1 (page
//   'Griffin 第 4、5 节 H800 对照协议', 'RG-LRU 的固定方程', says the same);
//   gate preparation is fused into the summary and replay kernels (no
//   pointwise intermediates in memory); the backward recomputes the gates,
//   runs the adjoint in reverse with resets as a = 0, forms per-(batch,
//   chunk) alpha partials and reduces them over batch and chunks to [D]; the
//   square-root derivative is truncated (capped at 1000 here).
//
// Layout: lanes run over channels, VM = 2 channels per lane, so each token
// costs one 32-bit load per input tensor per lane; a workgroup owns one chunk
// of one batch row and 256 * VM channels.
#include "common.hpp"

namespace lrs {
namespace {

constexpr int RG_VM = 2;
constexpr int RG_THREADS = 256;
// 1/(2 sqrt(u)) is capped at 1000: u is clamped below at 1/(4 * 1000^2).
constexpr float RG_SQRT_UMIN = 2.5e-7f;
constexpr float LOG2E = 1.4426950408889634f;

struct ChanConst {
    float k8;     // -8 softplus(alpha) log2(e): a = 2^(k8 g^a)
    float sp;     // softplus(alpha)
    float dsp;    // sigmoid(alpha) = d softplus / d alpha
};

__device__ __forceinline__ ChanConst chan_const(float alpha) {
    ChanConst k;
    const float sp = alpha > 20.f ? alpha + log1pf(expf(-alpha)) : log1pf(expf(alpha));
    k.sp = sp;
    k.k8 = -8.0f * sp * LOG2E;
    k.dsp = 1.0f / (1.0f + expf(-alpha));
    return k;
}

__device__ __forceinline__ float sigm(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * LOG2E));
}

struct Gate {
    float a, m, gx, ga;
};

// Gates of one channel at one token; rs = segment start.
__device__ __forceinline__ Gate gates(const ChanConst& k, float lx, float la, bool rs) {
    Gate g;
    g.gx = sigm(lx);
    g.ga = sigm(la);
    const float a = __builtin_amdgcn_exp2f(k.k8 * g.ga);
    const float u = fmaxf(fmaf(-a, a, 1.0f), 0.0f);
    g.a = rs ? 0.0f : a;
    g.m = rs ? 1.0f : __builtin_amdgcn_sqrtf(u);
    return g;
}

__device__ __forceinline__ float retention(const ChanConst& k, float la, bool rs) {
    return rs ? 0.0f : __builtin_amdgcn_exp2f(k.k8 * sigm(la));
}

__device__ __forceinline__ bool seg_start(const unsigned char* reset, size_t tok) {
    return reset != nullptr && reset[tok] != 0;
}

// ---------------------------------------------------------------- K11 ---
template <int K>
__global__ __launch_bounds__(RG_THREADS) void rglru_summary_kernel(
    int L, int D, int C, const uint32_t* __restrict__ x, const uint32_t* __restrict__ lx,
    const uint32_t* __restrict__ la, const float* __restrict__ alpha,
    const unsigned char* __restrict__ reset, float* __restrict__ summ) {
    const int d0 = (blockIdx.x * RG_THREADS + threadIdx.x) * RG_VM;
    const int c = blockIdx.y, b = blockIdx.z;
    if (d0 >= D) return;
    const int W = D / 2;  // words per row
    ChanConst k[RG_VM];
    float A[RG_VM], Bv[RG_VM];
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) { k[v] = chan_const(alpha[d0 + v]); A[v] = 1.f; Bv[v] = 0.f; }
    const int s = c * K;
    const int kc = min(K, L - s);
    const size_t tok0 = (size_t)b * L + s;
    const size_t w0 = tok0 * W + d0 / 2;
    auto step = [&](int i) {
        const bool rs = seg_start(reset, tok0 + i);
        const uint32_t xw = x[w0 + (size_t)i * W], lxw = lx[w0 + (size_t)i * W], law = la[w0 + (size_t)i * W];
        const float xv[2] = {bf16_lo(xw), bf16_hi(xw)};
        const float lxv[2] = {bf16_lo(lxw), bf16_hi(lxw)};
        const float lav[2] = {bf16_lo(law), bf16_hi(law)};
#pragma unroll
        for (int v = 0; v < RG_VM; ++v) {
            const Gate g = gates(k[v], lxv[v], lav[v], rs);
            A[v] *= g.a;
            Bv[v] = fmaf(g.a, Bv[v], xv[v] * g.gx * g.m);
        }
    };
    if (kc == K) {
#pragma unroll
        for (int i = 0; i < K; ++i) step(i);
    } else {
        for (int i = 0; i < kc; ++i) step(i);
    }
    float2* out = reinterpret_cast<float2*>(summ) + ((size_t)b * C + c) * D + d0;
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) out[v] = make_float2(A[v], Bv[v]);
}

// ---------------------------------------------------------------- K12 ---
template <int K, bool F32>
__global__ __launch_bounds__(RG_THREADS) void rglru_replay_kernel(
    int L, int D, int C, const uint32_t* __restrict__ x, const uint32_t* __restrict__ lx,
    const uint32_t* __restrict__ la, const float* __restrict__ alpha,
    const unsigned char* __restrict__ reset, const float* __restrict__ entries,
    void* __restrict__ y, float* __restrict__ h_final) {
    const int d0 = (blockIdx.x * RG_THREADS + threadIdx.x) * RG_VM;
    const int c = blockIdx.y, b = blockIdx.z;
    if (d0 >= D) return;
    const int W = D / 2;
    ChanConst k[RG_VM];
    float h[RG_VM];
    const float* ent = entries + ((size_t)b * C + c) * D + d0;
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) { k[v] = chan_const(alpha[d0 + v]); h[v] = ent[v]; }
    const int s = c * K;
    const int kc = min(K, L - s);
    const size_t tok0 = (size_t)b * L + s;
    const size_t w0 = tok0 * W + d0 / 2;
    auto step = [&](int i) {
        const bool rs = seg_start(reset, tok0 + i);
        const size_t wi = w0 + (size_t)i * W;
        const uint32_t xw = x[wi], lxw = lx[wi], law = la[wi];
        const float xv[2] = {bf16_lo(xw), bf16_hi(xw)};
        const float lxv[2] = {bf16_lo(lxw), bf16_hi(lxw)};
        const float lav[2] = {bf16_lo(law), bf16_hi(law)};
#pragma unroll
        for (int v = 0; v < RG_VM; ++v) {
            const Gate g = gates(k[v], lxv[v], lav[v], rs);
            h[v] = fmaf(g.a, h[v], xv[v] * g.gx * g.m);
        }
        if (F32) reinterpret_cast<float2*>(y)[wi] = make_float2(h[0], h[1]);
        else reinterpret_cast<uint32_t*>(y)[wi] = pack_bf16x2(h[0], h[1]);
    };
    if (kc == K) {
#pragma unroll
        for (int i = 0; i < K; ++i) step(i);
    } else {
        for (int i = 0; i < kc; ++i) step(i);
    }
    if (h_final && c == C - 1) {
#pragma unroll
        for (int v = 0; v < RG_VM; ++v) h_final[(size_t)b * D + d0 + v] = h[v];
    }
}

// ---------------------------------------------------------------- K13 ---
// Reverse summary: carry -> a_t (dy_t + carry) composed from the last token of
// the chunk to the first.
template <int K>
__global__ __launch_bounds__(RG_THREADS) void rglru_rev_summary_kernel(
    int L, int D, int C, const uint32_t* __restrict__ la, const float* __restrict__ alpha,
    const unsigned char* __restrict__ reset, const uint32_t* __restrict__ dy,
    float* __restrict__ summ) {
    const int d0 = (blockIdx.x * RG_THREADS + threadIdx.x) * RG_VM;
    const int c = blockIdx.y, b = blockIdx.z;
    if (d0 >= D) return;
    const int W = D / 2;
    ChanConst k[RG_VM];
    float A[RG_VM], Bv[RG_VM];
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) { k[v] = chan_const(alpha[d0 + v]); A[v] = 1.f; Bv[v] = 0.f; }
    const int s = c * K;
    const int kc = min(K, L - s);
    const size_t tok0 = (size_t)b * L + s;
    const size_t w0 = tok0 * W + d0 / 2;
    auto step = [&](int i) {
        const bool rs = seg_start(reset, tok0 + i);
        const size_t wi = w0 + (size_t)i * W;
        const uint32_t law = la[wi], gw = dy[wi];
        const float lav[2] = {bf16_lo(law), bf16_hi(law)};
        const float gv[2] = {bf16_lo(gw), bf16_hi(gw)};
#pragma unroll
        for (int v = 0; v < RG_VM; ++v) {
            const float a = retention(k[v], lav[v], rs);
            A[v] *= a;
            Bv[v] = a * (Bv[v] + gv[v]);
        }
    };
    if (kc == K) {
#pragma unroll
        for (int i = K - 1; i >= 0; --i) step(i);
    } else {
        for (int i = kc - 1; i >= 0; --i) step(i);
    }
    float2* out = reinterpret_cast<float2*>(summ) + ((size_t)b * C + c) * D + d0;
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) out[v] = make_float2(A[v], Bv[v]);
}

// ---------------------------------------------------------------- K14 ---
// Backward replay: recompute h over the chunk from its entry state (keeping
// h_{t-1} and the raw input words in registers), then run the adjoint in
// reverse from the chunk's carry-in, regenerating the gates.
template <int K, bool F32>
__global__ __launch_bounds__(RG_THREADS) void rglru_bwd_replay_kernel(
    int L, int D, int C, const uint32_t* __restrict__ x, const uint32_t* __restrict__ lx,
    const uint32_t* __restrict__ la, const float* __restrict__ alpha,
    const unsigned char* __restrict__ reset, const float* __restrict__ entries,
    const float* __restrict__ carry_in, const uint32_t* __restrict__ dy, void* __restrict__ dx,
    void* __restrict__ dlx, void* __restrict__ dla, float* __restrict__ dh0,
    float* __restrict__ alpha_part) {
    const int d0 = (blockIdx.x * RG_THREADS + threadIdx.x) * RG_VM;
    const int c = blockIdx.y, b = blockIdx.z;
    if (d0 >= D) return;
    const int W = D / 2;
    ChanConst k[RG_VM];
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) k[v] = chan_const(alpha[d0 + v]);
    const int s = c * K;
    const int kc = min(K, L - s);
    const size_t tok0 = (size_t)b * L + s;
    const size_t w0 = tok0 * W + d0 / 2;
    const size_t cidx = ((size_t)b * C + c) * D + d0;

    uint32_t xs[K], lxs[K], las[K];
    float hp[K][RG_VM];
    {
        float h[RG_VM];
#pragma unroll
        for (int v = 0; v < RG_VM; ++v) h[v] = entries[cidx + v];
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (i < kc) {
                const bool rs = seg_start(reset, tok0 + i);
                const size_t wi = w0 + (size_t)i * W;
                xs[i] = x[wi];
                lxs[i] = lx[wi];
                las[i] = la[wi];
                const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
                const float lxv[2] = {bf16_lo(lxs[i]), bf16_hi(lxs[i])};
                const float lav[2] = {bf16_lo(las[i]), bf16_hi(las[i])};
#pragma unroll
                for (int v = 0; v < RG_VM; ++v) {
                    hp[i][v] = h[v];
                    const Gate g = gates(k[v], lxv[v], lav[v], rs);
                    h[v] = fmaf(g.a, h[v], xv[v] * g.gx * g.m);
                }
            }
        }
    }
    float carry[RG_VM], acc_al[RG_VM];
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) { carry[v] = carry_in[cidx + v]; acc_al[v] = 0.f; }
#pragma unroll
    for (int i = K - 1; i >= 0; --i) {
        if (i < kc) {
            const bool rs = seg_start(reset, tok0 + i);
            const size_t wi = w0 + (size_t)i * W;
            const uint32_t gw = dy[wi];
            const float gv[2] = {bf16_lo(gw), bf16_hi(gw)};
            const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
            const float lxv[2] = {bf16_lo(lxs[i]), bf16_hi(lxs[i])};
            const float lav[2] = {bf16_lo(las[i]), bf16_hi(las[i])};
            float ox[RG_VM], olx[RG_VM], ola[RG_VM];
#pragma unroll
            for (int v = 0; v < RG_VM; ++v) {
                const Gate gt = gates(k[v], lxv[v], lav[v], rs);
                const float g = gv[v] + carry[v];
                ox[v] = g * gt.gx * gt.m;
                olx[v] = ox[v] * xv[v] * (1.0f - gt.gx);
                float abar = 0.f;
                if (!rs) {
                    const float u = fmaxf(fmaf(-gt.a, gt.a, 1.0f), RG_SQRT_UMIN);
                    const float dm_da = -gt.a * __builtin_amdgcn_rsqf(u);
                    abar = g * fmaf(xv[v] * gt.gx, dm_da, hp[i][v]);
                }
                // d a / d l^a = a (-8 sp) g^a (1 - g^a); d a / d alpha = a (-8 g^a) sigmoid(alpha)
                const float ag = abar * gt.a * gt.ga;
                ola[v] = ag * (-8.0f * k[v].sp) * (1.0f - gt.ga);
                acc_al[v] += ag;
                carry[v] = gt.a * g;
            }
            if (F32) {
                reinterpret_cast<float2*>(dx)[wi] = make_float2(ox[0], ox[1]);
                reinterpret_cast<float2*>(dlx)[wi] = make_float2(olx[0], olx[1]);
                reinterpret_cast<float2*>(dla)[wi] = make_float2(ola[0], ola[1]);
            } else {
                reinterpret_cast<uint32_t*>(dx)[wi] = pack_bf16x2(ox[0], ox[1]);
                reinterpret_cast<uint32_t*>(dlx)[wi] = pack_bf16x2(olx[0], olx[1]);
                reinterpret_cast<uint32_t*>(dla)[wi] = pack_bf16x2(ola[0], ola[1]);
            }
        }
    }
#pragma unroll
    for (int v = 0; v < RG_VM; ++v) alpha_part[cidx + v] = acc_al[v] * (-8.0f * k[v].dsp);
    if (dh0 && c == 0) {
#pragma unroll
        for (int v = 0; v < RG_VM; ++v) dh0[(size_t)b * D + d0 + v] = carry[v];
    }
}

// ---------------------------------------------------------------- K15 ---
// d alpha = sum over batch rows and chunks of the per-chunk partials, FP64,
// fixed order.
__global__ __launch_bounds__(256) void rglru_alpha_reduce_kernel(
    int D, int nchunks, const float* __restrict__ part, float* __restrict__ dalpha) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= D) return;
    double s = 0.0;
    for (int i = 0; i < nchunks; ++i) s += part[(size_t)i * D + d];
    dalpha[d] = (float)s;
}

inline dim3 rg_grid(int D, const Chunking& ch) {
    return dim3((unsigned)ceil_div(ceil_div(D, RG_VM), RG_THREADS), ch.C, ch.B);
}

}  // namespace

hipError_t launch_rglru_summary(const RglruParams& p, const Chunking& ch, float* summ, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
#define RG_SUM(KK)                                                                                  \
    LRS_LAUNCH(K_RGLRU_SUMMARY, rglru_summary_kernel<KK>, grid, dim3(RG_THREADS), 0, s, p.L, p.D, \
               ch.C, (const uint32_t*)p.x, (const uint32_t*)p.lx, (const uint32_t*)p.la, p.alpha,  \
               p.reset, summ)
    if (ch.K == 32) RG_SUM(32); else RG_SUM(16);
#undef RG_SUM
    return hipGetLastError();
}

hipError_t launch_rglru_replay(const RglruParams& p, const Chunking& ch, const float* entries, void* y,
                               int y_f32, float* h_final, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
#define RG_REP(KK, FF)                                                                                 \
    LRS_LAUNCH(K_RGLRU_REPLAY, (rglru_replay_kernel<KK, FF>), grid, dim3(RG_THREADS), 0, s, p.L, p.D, \
               ch.C, (const uint32_t*)p.x, (const uint32_t*)p.lx, (const uint32_t*)p.la, p.alpha,     \
               p.reset, entries, y, h_final)
    if (ch.K == 32) { if (y_f32) RG_REP(32, true); else RG_REP(32, false); }
    else { if (y_f32) RG_REP(16, true); else RG_REP(16, false); }
#undef RG_REP
    return hipGetLastError();
}

hipError_t launch_rglru_rev_summary(const RglruParams& p, const Chunking& ch, const void* dy,
                                    float* summ, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
#define RG_RSUM(KK)                                                                                   \
    LRS_LAUNCH(K_RGLRU_REV_SUMMARY, rglru_rev_summary_kernel<KK>, grid, dim3(RG_THREADS), 0, s, p.L, \
               p.D, ch.C, (const uint32_t*)p.la, p.alpha, p.reset, (const uint32_t*)dy, summ)
    if (ch.K == 32) RG_RSUM(32); else RG_RSUM(16);
#undef RG_RSUM
    return hipGetLastError();
}

hipError_t launch_rglru_bwd_replay(const RglruParams& p, const Chunking& ch, const float* entries,
                                   const float* carry_in, const void* dy, void* dx, void* dlx, void* dla,
                                   int g_f32, float* dh0, float* alpha_part, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
#define RG_BWD(KK, FF)                                                                                \
    LRS_LAUNCH(K_RGLRU_BWD_REPLAY, (rglru_bwd_replay_kernel<KK, FF>), grid, dim3(RG_THREADS), 0, s,  \
               p.L, p.D, ch.C, (const uint32_t*)p.x, (const uint32_t*)p.lx, (const uint32_t*)p.la,   \
               p.alpha, p.reset, entries, carry_in, (const uint32_t*)dy, dx, dlx, dla, dh0,          \
               alpha_part)
    if (ch.K == 32) { if (g_f32) RG_BWD(32, true); else RG_BWD(32, false); }
    else { if (g_f32) RG_BWD(16, true); else RG_BWD(16, false); }
#undef RG_BWD
    return hipGetLastError();
}

hipError_t launch_rglru_alpha_reduce(const RglruParams& p, const Chunking& ch, const float* alpha_part,
                                     float* dalpha, hipStream_t s) {
    LRS_LAUNCH(K_RGLRU_ALPHA_REDUCE, rglru_alpha_reduce_kernel, dim3((unsigned)ceil_div(p.D, 256)),
               dim3(256), 0, s, p.D, ch.B * ch.C, alpha_part, dalpha);
    return hipGetLastError();
}

}  // namespace lrs
