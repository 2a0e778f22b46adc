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
// Layout: lanes run over channel pairs (one 32-bit word of each BF16 tensor
// per lane and token, so a wave reads 256 contiguous bytes of a row); a
// workgroup owns one chunk of one batch row and 512 channels.  Every chunk
// but a ragged last one is loaded branch-free from a uniform row base plus
// a 32-bit lane offset; the last one takes a guarded instance of the same
// code.
//
// Special functions per channel and token: both sigmoids share one
// reciprocal, 1/((1+e^-lx)(1+e^-la)), and one reciprocal square root gives
// both sqrt(u) = u rsq(u) and the capped derivative rsq(max(u, u_min)) =
// min(rsq(u), rsq(u_min)).
#include "common.hpp"

namespace lrs {
namespace {

constexpr int RG_THREADS = 256;
#ifndef LRS_RG_BWD_H
#define LRS_RG_BWD_H 16
#endif
#ifndef LRS_RG_BWD_KEEP
#define LRS_RG_BWD_KEEP 0
#endif
constexpr int RG_BWD_H = LRS_RG_BWD_H;       // backward sub-chunk length
constexpr bool RG_BWD_KEEP = LRS_RG_BWD_KEEP; // keep forward gates live (vs recompute)
constexpr int RG_CH = 2 * RG_THREADS;     // channels per workgroup
// 1/(2 sqrt(u)) is capped at 1000: the reciprocal square root used for the
// derivative is capped at 2000 = rsq(2.5e-7).
constexpr float RG_RSQ_CAP = 2000.0f;
constexpr float LOG2E = 1.4426950408889634f;
// e^-v is formed as 2^min(-v log2 e, 57.7) (v >= -40): the product of two
// such factors stays below FP32 overflow; sigmoid(-40) ~ 4e-18 absorbs it.
constexpr float RG_EXP_ARG_MAX = 57.7f;

struct ChanConst {
    float k8;     // -8 softplus(alpha) log2(e): a = 2^(k8 g^a)
    float sp8;    // -8 softplus(alpha)
    float dsp8;   // -8 sigmoid(alpha) = -8 d softplus / d alpha
};

__device__ __forceinline__ ChanConst chan_const(float alpha) {
    ChanConst k;
    const float sp = alpha > 20.f ? alpha + log1pf(expf(-alpha)) : log1pf(expf(alpha));
    k.sp8 = -8.0f * sp;
    k.k8 = k.sp8 * LOG2E;
    k.dsp8 = -8.0f / (1.0f + expf(-alpha));
    return k;
}

__device__ __forceinline__ float neg_exp(float v) {
    return __builtin_amdgcn_exp2f(fminf(-v * LOG2E, RG_EXP_ARG_MAX));
}

__device__ __forceinline__ float sigm(float v) { return __builtin_amdgcn_rcpf(1.0f + neg_exp(v)); }

struct Gate {
    float gx, ga;   // sigmoid(l^x), sigmoid(l^a)
    float a0;       // retention before a reset
    float a, m;     // retention and normalization after a reset
    float r;        // rsq(1 - a0^2) (infinite-free)
};

// Gates of one channel at one token; rs = segment start.
__device__ __forceinline__ Gate gates(const ChanConst& k, float lx, float la, bool rs) {
    Gate g;
    const float px = 1.0f + neg_exp(lx), pa = 1.0f + neg_exp(la);
    const float q = __builtin_amdgcn_rcpf(px * pa);
    g.gx = q * pa;
    g.ga = q * px;
    g.a0 = __builtin_amdgcn_exp2f(k.k8 * g.ga);
    // 1 - a^2 >= 0 exactly (a <= 1), so the FMA result is >= 0; the floor only
    // keeps rsq finite at a = 1, where u rsq(u) is then 0 as it must be
    const float u = fmaxf(fmaf(-g.a0, g.a0, 1.0f), 1e-30f);
    g.r = __builtin_amdgcn_rsqf(u);
    g.a = rs ? 0.0f : g.a0;
    g.m = rs ? 1.0f : u * g.r;
    return g;
}

// retention with a segment start applied as a multiplier, so that no uniform
// branch splits the token loop around the special functions
__device__ __forceinline__ float retention(const ChanConst& k, float la, bool rs) {
    return __builtin_amdgcn_exp2f(k.k8 * sigm(la)) * (rs ? 0.0f : 1.0f);
}

// Segment-start flags of a chunk as a wave-uniform bit mask (bit i = token
// i): lane i reads flag i and a ballot gathers them, one load for the chunk,
// so the token loop has no load or branch on the flag array.  Called at
// kernel entry, before any lane leaves, by all 64 lanes of the wave.
template <int K>
__device__ __forceinline__ uint32_t reset_mask(const unsigned char* reset, size_t tok0, int kc) {
    static_assert(K <= 32, "one mask word per chunk");
    if (!reset) return 0;
    const int l = threadIdx.x & 63;
    const bool f = l < kc && reset[tok0 + l] != 0;
    return (uint32_t)__ballot(f);
}

__device__ __forceinline__ bool bit(uint32_t m, int i) { return (m >> i) & 1u; }

struct RgIn {
    int L, W;     // W = D / 2 words per row
    const uint32_t* x;
    const uint32_t* lx;
    const uint32_t* la;
    const unsigned char* reset;
};

// word of token i of the chunk starting at token tok0: uniform row, lane offset
__device__ __forceinline__ uint32_t word(const uint32_t* t, size_t tok0, int i, int W, int lw) {
    return (t + (tok0 + i) * (size_t)W)[lw];
}

// ---------------------------------------------------------------- summary
template <int K, bool FULL>
__device__ __forceinline__ void rg_summary_chunk(const RgIn& in, const ChanConst (&k)[2], size_t tok0,
                                                 int lw, int kc, uint32_t rm, float (&A)[2], float (&Bv)[2]) {
    const int kq = FULL ? K : opaque(kc);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const uint32_t xw = word(in.x, tok0, i, in.W, lw);
            const uint32_t lxw = word(in.lx, tok0, i, in.W, lw);
            const uint32_t law = word(in.la, tok0, i, in.W, lw);
            const float xv[2] = {bf16_lo(xw), bf16_hi(xw)};
            const float lxv[2] = {bf16_lo(lxw), bf16_hi(lxw)};
            const float lav[2] = {bf16_lo(law), bf16_hi(law)};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate g = gates(k[v], lxv[v], lav[v], rs);
                A[v] *= g.a;
                Bv[v] = fmaf(g.a, Bv[v], xv[v] * g.gx * g.m);
            }
        }
    }
}

template <int K>
__global__ __launch_bounds__(RG_THREADS) void rglru_summary_kernel(RgIn in, int C,
                                                                   const float* __restrict__ alpha,
                                                                   float* __restrict__ summ) {
    const int lw = blockIdx.x * RG_THREADS + threadIdx.x;
    const int c = blockIdx.y, b = blockIdx.z;
    const size_t tok0 = (size_t)b * in.L + (size_t)c * K;
    const int kc = min(K, in.L - c * K);
    const uint32_t rm = reset_mask<K>(in.reset, tok0, kc);
    if (lw >= in.W) return;
    const ChanConst k[2] = {chan_const(alpha[2 * lw]), chan_const(alpha[2 * lw + 1])};
    float A[2] = {1.f, 1.f}, Bv[2] = {0.f, 0.f};
    if (kc == K) rg_summary_chunk<K, true>(in, k, tok0, lw, K, rm, A, Bv);
    else rg_summary_chunk<K, false>(in, k, tok0, lw, kc, rm, A, Bv);
    float4* out = reinterpret_cast<float4*>(summ + (((size_t)b * C + c) * in.W + lw) * 4);
    *out = make_float4(A[0], Bv[0], A[1], Bv[1]);
}

// ----------------------------------------------------------------- replay
template <int K, bool F32, bool FULL>
__device__ __forceinline__ void rg_replay_chunk(const RgIn& in, const ChanConst (&k)[2], size_t tok0,
                                                int lw, int kc, uint32_t rm, float (&h)[2], void* __restrict__ y) {
    const int kq = FULL ? K : opaque(kc);
    // all loads of the chunk ahead of its stores (y may not be assumed
    // disjoint from the inputs held in the struct)
    uint32_t xs[K], lxs[K], las[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (FULL || i < kq) {
            xs[i] = word(in.x, tok0, i, in.W, lw);
            lxs[i] = word(in.lx, tok0, i, in.W, lw);
            las[i] = word(in.la, tok0, i, in.W, lw);
        }
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
            const float lxv[2] = {bf16_lo(lxs[i]), bf16_hi(lxs[i])};
            const float lav[2] = {bf16_lo(las[i]), bf16_hi(las[i])};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate g = gates(k[v], lxv[v], lav[v], rs);
                h[v] = fmaf(g.a, h[v], xv[v] * g.gx * g.m);
            }
            const size_t row = (tok0 + i) * (size_t)in.W;
            if (F32) out_f32x2(reinterpret_cast<float2*>(y) + row + lw, h[0], h[1]);
            else out_u32(reinterpret_cast<uint32_t*>(y) + row + lw, pack_bf16x2(h[0], h[1]));
        }
    }
}

template <int K, bool F32>
__global__ __launch_bounds__(RG_THREADS) void rglru_replay_kernel(RgIn in, int C,
                                                                  const float* __restrict__ alpha,
                                                                  const float* __restrict__ entries,
                                                                  void* __restrict__ y,
                                                                  float* __restrict__ h_final) {
    const int lw = blockIdx.x * RG_THREADS + threadIdx.x;
    const int c = blockIdx.y, b = blockIdx.z;
    const size_t tok0 = (size_t)b * in.L + (size_t)c * K;
    const int kc = min(K, in.L - c * K);
    const uint32_t rm = reset_mask<K>(in.reset, tok0, kc);
    if (lw >= in.W) return;
    const ChanConst k[2] = {chan_const(alpha[2 * lw]), chan_const(alpha[2 * lw + 1])};
    const float2 e = reinterpret_cast<const float2*>(entries)[((size_t)b * C + c) * in.W + lw];
    float h[2] = {e.x, e.y};
    if (kc == K) rg_replay_chunk<K, F32, true>(in, k, tok0, lw, K, rm, h, y);
    else rg_replay_chunk<K, F32, false>(in, k, tok0, lw, kc, rm, h, y);
    if (h_final && c == C - 1)
        reinterpret_cast<float2*>(h_final)[(size_t)b * in.W + lw] = make_float2(h[0], h[1]);
}

// -------------------------------------------------------- reverse summary
// carry -> a_t (dy_t + carry), composed from the last token of the chunk to
// the first: (A, B) with carry_before = A carry_after + B.
template <int K, bool FULL>
__device__ __forceinline__ void rg_rev_summary_chunk(const RgIn& in, const ChanConst (&k)[2],
                                                     const uint32_t* __restrict__ dy, size_t tok0,
                                                     int lw, int kc, uint32_t rm, float (&A)[2],
                                                     float (&Bv)[2]) {
    const int kq = FULL ? K : opaque(kc);
#pragma unroll
    for (int i = K - 1; i >= 0; --i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const uint32_t law = word(in.la, tok0, i, in.W, lw);
            const uint32_t gw = word(dy, tok0, i, in.W, lw);
            const float lav[2] = {bf16_lo(law), bf16_hi(law)};
            const float gv[2] = {bf16_lo(gw), bf16_hi(gw)};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const float a = retention(k[v], lav[v], rs);
                A[v] *= a;
                Bv[v] = a * (Bv[v] + gv[v]);
            }
        }
    }
}

template <int K>
__global__ __launch_bounds__(RG_THREADS) void rglru_rev_summary_kernel(RgIn in, int C,
                                                                       const float* __restrict__ alpha,
                                                                       const uint32_t* __restrict__ dy,
                                                                       float* __restrict__ summ) {
    const int lw = blockIdx.x * RG_THREADS + threadIdx.x;
    const int c = blockIdx.y, b = blockIdx.z;
    const size_t tok0 = (size_t)b * in.L + (size_t)c * K;
    const int kc = min(K, in.L - c * K);
    const uint32_t rm = reset_mask<K>(in.reset, tok0, kc);
    if (lw >= in.W) return;
    const ChanConst k[2] = {chan_const(alpha[2 * lw]), chan_const(alpha[2 * lw + 1])};
    float A[2] = {1.f, 1.f}, Bv[2] = {0.f, 0.f};
    if (kc == K) rg_rev_summary_chunk<K, true>(in, k, dy, tok0, lw, K, rm, A, Bv);
    else rg_rev_summary_chunk<K, false>(in, k, dy, tok0, lw, kc, rm, A, Bv);
    float4* out = reinterpret_cast<float4*>(summ + (((size_t)b * C + c) * in.W + lw) * 4);
    *out = make_float4(A[0], Bv[0], A[1], Bv[1]);
}

// -------------------------------------------------------- backward replay
// The chunk is handled H tokens at a time, last sub-chunk first.  For each
// sub-chunk the forward is recomputed from a checkpoint (the state entering
// the sub-chunk, found by one forward pass over the earlier sub-chunks),
// keeping the three input words in registers and h_{t-1} in the lane's own
// LDS slots; then the adjoint runs back over it, regenerating the gates,
// from the cotangent carried in.  The history in LDS keeps the kernel at
// 4 waves per SIMD (123 VGPRs; in registers it took 139, 3 waves).
struct RgBwdOut {
    const uint32_t* dy;
    void* dx;
    void* dlx;
    void* dla;
};

template <int H, bool F32, bool FULL>
__device__ __forceinline__ void rg_bwd_sub(const RgIn& in, const ChanConst (&k)[2], const RgBwdOut& o,
                                           size_t tok0, int lw, int kq, uint32_t rm,
                                           const float (&h_in)[2], float (&carry)[2], float (&acc)[2],
                                           float2* hist) {
    uint32_t xs[H], lxs[H], las[H], gws[H];
    float h[2] = {h_in[0], h_in[1]};
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (FULL || i < kq) {
            xs[i] = word(in.x, tok0, i, in.W, lw);
            lxs[i] = word(in.lx, tok0, i, in.W, lw);
            las[i] = word(in.la, tok0, i, in.W, lw);
            gws[i] = word(o.dy, tok0, i, in.W, lw);
        }
    }
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
            const float lxv[2] = {bf16_lo(lxs[i]), bf16_hi(lxs[i])};
            const float lav[2] = {bf16_lo(las[i]), bf16_hi(las[i])};
            hist[i * 64] = make_float2(h[0], h[1]);
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate g = gates(k[v], lxv[v], lav[v], rs);
                h[v] = fmaf(g.a, h[v], xv[v] * g.gx * g.m);
            }
        }
    }
    asm volatile("" ::: "memory");  // read the history back from LDS, not from registers
#pragma unroll
    for (int i = H - 1; i >= 0; --i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const float gv[2] = {bf16_lo(gws[i]), bf16_hi(gws[i])};
            const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
            // the gates are evaluated again rather than kept from the forward
            // pass: six live values per token and channel would not fit
            const uint32_t lxw = RG_BWD_KEEP ? lxs[i] : opaque_v(lxs[i]);
            const uint32_t law = RG_BWD_KEEP ? las[i] : opaque_v(las[i]);
            const float lxv[2] = {bf16_lo(lxw), bf16_hi(lxw)};
            const float lav[2] = {bf16_lo(law), bf16_hi(law)};
            const float2 hv = hist[i * 64];
            const float hpv[2] = {hv.x, hv.y};
            float ox[2], olx[2], ola[2];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate gt = gates(k[v], lxv[v], lav[v], rs);
                const float g = gv[v] + carry[v];
                const float xg = xv[v] * gt.gx;
                ox[v] = g * gt.gx * gt.m;
                olx[v] = g * xg * gt.m * (1.0f - gt.gx);
                // d h / d a = h_{t-1} + x g^x dm/da, dm/da = -a / sqrt(u) (capped);
                // zero at a segment start, where a and m are constants
                const float dm_da = -gt.a0 * fminf(gt.r, RG_RSQ_CAP);
                const float abar = rs ? 0.0f : g * fmaf(xg, dm_da, hpv[v]);
                // d a / d l^a = a (-8 sp) g^a (1 - g^a); d a / d alpha = a g^a (-8 sigmoid(alpha))
                const float ag = abar * gt.a0 * gt.ga;
                ola[v] = ag * k[v].sp8 * (1.0f - gt.ga);
                acc[v] += ag;
                carry[v] = gt.a * g;
            }
            const size_t row = (tok0 + i) * (size_t)in.W;
            if (F32) {
                out_f32x2(reinterpret_cast<float2*>(o.dx) + row + lw, ox[0], ox[1]);
                out_f32x2(reinterpret_cast<float2*>(o.dlx) + row + lw, olx[0], olx[1]);
                out_f32x2(reinterpret_cast<float2*>(o.dla) + row + lw, ola[0], ola[1]);
            } else {
                out_u32(reinterpret_cast<uint32_t*>(o.dx) + row + lw, pack_bf16x2(ox[0], ox[1]));
                out_u32(reinterpret_cast<uint32_t*>(o.dlx) + row + lw, pack_bf16x2(olx[0], olx[1]));
                out_u32(reinterpret_cast<uint32_t*>(o.dla) + row + lw, pack_bf16x2(ola[0], ola[1]));
            }
        }
    }
}

// state after `n` tokens (n <= H, guarded when not FULL) from h
template <int H, bool FULL>
__device__ __forceinline__ void rg_advance(const RgIn& in, const ChanConst (&k)[2], size_t tok0, int lw,
                                           int kq, uint32_t rm, float (&h)[2]) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const uint32_t xw = word(in.x, tok0, i, in.W, lw);
            const uint32_t lxw = word(in.lx, tok0, i, in.W, lw);
            const uint32_t law = word(in.la, tok0, i, in.W, lw);
            const float xv[2] = {bf16_lo(xw), bf16_hi(xw)};
            const float lxv[2] = {bf16_lo(lxw), bf16_hi(lxw)};
            const float lav[2] = {bf16_lo(law), bf16_hi(law)};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate g = gates(k[v], lxv[v], lav[v], rs);
                h[v] = fmaf(g.a, h[v], xv[v] * g.gx * g.m);
            }
        }
    }
}

template <int K, int H, bool F32, bool FULL>
__device__ __forceinline__ void rg_bwd_chunk(const RgIn& in, const ChanConst (&k)[2], const RgBwdOut& o,
                                             size_t tok0, int lw, int kc, uint32_t rm,
                                             const float (&h0)[2], float (&carry)[2], float (&acc)[2],
                                             float2* hist) {
    constexpr int NS = K / H;
    const int kq = FULL ? K : opaque(kc);
    float ck[NS][2];
    float h[2] = {h0[0], h0[1]};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        ck[s][0] = h[0];
        ck[s][1] = h[1];
        if (s + 1 < NS) rg_advance<H, FULL>(in, k, tok0 + s * H, lw, kq - s * H, rm >> (s * H), h);
    }
#pragma unroll
    for (int s = NS - 1; s >= 0; --s)
        rg_bwd_sub<H, F32, FULL>(in, k, o, tok0 + s * H, lw, kq - s * H, rm >> (s * H), ck[s], carry, acc,
                                 hist);
}

#ifndef LRS_RG_BWD_WPE
#define LRS_RG_BWD_WPE 1
#endif
template <int K, int H, bool F32>
__global__ __launch_bounds__(RG_THREADS) __attribute__((amdgpu_waves_per_eu(LRS_RG_BWD_WPE, 8))) void rglru_bwd_replay_kernel(
    RgIn in, int C, const float* __restrict__ alpha, const float* __restrict__ entries,
    const float* __restrict__ carry_in, RgBwdOut o, float* __restrict__ dh0,
    float* __restrict__ alpha_part) {
    const int lw = blockIdx.x * RG_THREADS + threadIdx.x;
    const int c = blockIdx.y, b = blockIdx.z;
    const size_t tok0 = (size_t)b * in.L + (size_t)c * K;
    const int kc = min(K, in.L - c * K);
    const uint32_t rm = reset_mask<K>(in.reset, tok0, kc);
    if (lw >= in.W) return;
    const ChanConst k[2] = {chan_const(alpha[2 * lw]), chan_const(alpha[2 * lw + 1])};
    const size_t cw = ((size_t)b * C + c) * in.W + lw;
    const float2 e = reinterpret_cast<const float2*>(entries)[cw];
    const float2 ci = reinterpret_cast<const float2*>(carry_in)[cw];
    const float h0[2] = {e.x, e.y};
    float carry[2] = {ci.x, ci.y}, acc[2] = {0.f, 0.f};
    // each lane's h_{t-1} history of a sub-chunk, [wave][token][lane]
    __shared__ float2 hist_all[RG_THREADS / 64][H][64];
    float2* hist = &hist_all[threadIdx.x >> 6][0][threadIdx.x & 63];
    if (kc == K) rg_bwd_chunk<K, H, F32, true>(in, k, o, tok0, lw, K, rm, h0, carry, acc, hist);
    else rg_bwd_chunk<K, H, F32, false>(in, k, o, tok0, lw, kc, rm, h0, carry, acc, hist);
    reinterpret_cast<float2*>(alpha_part)[cw] = make_float2(acc[0] * k[0].dsp8, acc[1] * k[1].dsp8);
    if (dh0 && c == 0) reinterpret_cast<float2*>(dh0)[(size_t)b * in.W + lw] = make_float2(carry[0], carry[1]);
}

// ------------------------------------------------------ alpha reduction
// d alpha = the sum of the B*C per-chunk partial rows, in one launch: a
// workgroup owns AR_COLS columns and splits the rows over AR_SG thread
// groups; group sg adds rows sg, sg + AR_SG, ... in FP64 and in order,
// AR_NB of them requested at once, and the group sums are added in group
// order through LDS, AR_L2 at a time.  The result depends on the shape alone.
constexpr int AR_COLS = 16;
constexpr int AR_SG = 64;
constexpr int AR_THREADS = AR_COLS * AR_SG;
constexpr int AR_NB = 16;
constexpr int AR_L2 = 8;

__global__ __launch_bounds__(AR_THREADS) void rglru_alpha_kernel(int R, int D, const float* __restrict__ part,
                                                                 float* __restrict__ dalpha) {
    __shared__ double g1[AR_SG][AR_COLS];
    __shared__ double g2[AR_SG / AR_L2][AR_COLS];
    const int sg = threadIdx.x / AR_COLS, cl = threadIdx.x - sg * AR_COLS;
    const int c0 = blockIdx.x * AR_COLS;
    const int col = min(c0 + cl, D - 1);
    double acc = 0.0;
    for (int r0 = sg; r0 < R; r0 += AR_SG * AR_NB) {
        float v[AR_NB];
#pragma unroll
        for (int k = 0; k < AR_NB; ++k) v[k] = part[(size_t)min(r0 + k * AR_SG, R - 1) * D + col];
#pragma unroll
        for (int k = 0; k < AR_NB; ++k) acc += r0 + k * AR_SG < R ? (double)v[k] : 0.0;
    }
    g1[sg][cl] = acc;
    __syncthreads();
    if (sg < AR_SG / AR_L2) {
        double t = 0.0;
#pragma unroll
        for (int g = 0; g < AR_L2; ++g) t += g1[sg * AR_L2 + g][cl];
        g2[sg][cl] = t;
    }
    __syncthreads();
    if (sg == 0 && c0 + cl < D) {
        double t = 0.0;
#pragma unroll
        for (int g = 0; g < AR_SG / AR_L2; ++g) t += g2[g][cl];
        dalpha[col] = (float)t;
    }
}

inline dim3 rg_grid(int D, const Chunking& ch) {
    return dim3((unsigned)ceil_div(D, RG_CH), ch.C, ch.B);
}

inline RgIn rg_in(const RglruParams& p) {
    return RgIn{p.L, p.D / 2, (const uint32_t*)p.x, (const uint32_t*)p.lx, (const uint32_t*)p.la, p.reset};
}

}  // namespace

hipError_t launch_rglru_summary(const RglruParams& p, const Chunking& ch, float* summ, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
    const RgIn in = rg_in(p);
    if (ch.K == 32)
        LRS_LAUNCH(K_RGLRU_SUMMARY, rglru_summary_kernel<32>, grid, dim3(RG_THREADS), 0, s, in, ch.C, p.alpha, summ);
    else
        LRS_LAUNCH(K_RGLRU_SUMMARY, rglru_summary_kernel<16>, grid, dim3(RG_THREADS), 0, s, in, ch.C, p.alpha, summ);
    return hipGetLastError();
}

hipError_t launch_rglru_replay(const RglruParams& p, const Chunking& ch, const float* entries, void* y,
                               int y_f32, float* h_final, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
    const RgIn in = rg_in(p);
#define RG_REP(KK, FF)                                                                                  \
    LRS_LAUNCH(K_RGLRU_REPLAY, (rglru_replay_kernel<KK, FF>), grid, dim3(RG_THREADS), 0, s, in, ch.C, \
               p.alpha, entries, y, h_final)
    if (ch.K == 32) { if (y_f32) RG_REP(32, true); else RG_REP(32, false); }
    else { if (y_f32) RG_REP(16, true); else RG_REP(16, false); }
#undef RG_REP
    return hipGetLastError();
}

hipError_t launch_rglru_rev_summary(const RglruParams& p, const Chunking& ch, const void* dy,
                                    float* summ, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
    const RgIn in = rg_in(p);
    if (ch.K == 32)
        LRS_LAUNCH(K_RGLRU_REV_SUMMARY, rglru_rev_summary_kernel<32>, grid, dim3(RG_THREADS), 0, s, in, ch.C,
                   p.alpha, (const uint32_t*)dy, summ);
    else
        LRS_LAUNCH(K_RGLRU_REV_SUMMARY, rglru_rev_summary_kernel<16>, grid, dim3(RG_THREADS), 0, s, in, ch.C,
                   p.alpha, (const uint32_t*)dy, summ);
    return hipGetLastError();
}

hipError_t launch_rglru_bwd_replay(const RglruParams& p, const Chunking& ch, const float* entries,
                                   const float* carry_in, const void* dy, void* dx, void* dlx, void* dla,
                                   int g_f32, float* dh0, float* alpha_part, hipStream_t s) {
    const dim3 grid = rg_grid(p.D, ch);
    const RgIn in = rg_in(p);
    const RgBwdOut o{(const uint32_t*)dy, dx, dlx, dla};
#define RG_BWD(KK, FF)                                                                                  \
    LRS_LAUNCH(K_RGLRU_BWD_REPLAY, (rglru_bwd_replay_kernel<KK, RG_BWD_H, FF>), grid, dim3(RG_THREADS), 0, s, \
               in, ch.C, p.alpha, entries, carry_in, o, dh0, alpha_part)
    if (ch.K == 32) { if (g_f32) RG_BWD(32, true); else RG_BWD(32, false); }
    else { if (g_f32) RG_BWD(16, true); else RG_BWD(16, false); }
#undef RG_BWD
    return hipGetLastError();
}

hipError_t launch_rglru_alpha_reduce(const RglruParams& p, const Chunking& ch, const float* alpha_part,
                                     float* dalpha, hipStream_t s) {
    LRS_LAUNCH(K_RGLRU_ALPHA, rglru_alpha_kernel, dim3((unsigned)ceil_div(p.D, AR_COLS)), dim3(AR_THREADS), 0, s,
               ch.B * ch.C, p.D, alpha_part, dalpha);
    return hipGetLastError();
}

}  // namespace lrs
