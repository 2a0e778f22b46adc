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
// per lane and token, so a wave reads 256 contiguous bytes of a row).  On
// the single-pass path (K = 16, groups of up to 16 chunks) a workgroup owns
// one group of chunks, one wave per chunk, and 64 channel pairs, and the
// groups hand states to each other; on the three-launch path a workgroup
// owns one chunk of one batch row and 512 channels, every chunk but a
// ragged last one loaded branch-free from a uniform row base plus a 32-bit
// lane offset, the last one by a guarded instance of the same code.
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

// Gates of one channel at one token; rs = segment start.  KNOWN: the
// retention a0 was formed earlier from the same inputs and is passed in.
template <bool KNOWN = false>
__device__ __forceinline__ Gate gates(const ChanConst& k, float lx, float la, bool rs, float a0 = 0.f) {
    Gate g;
    const float px = 1.0f + neg_exp(lx), pa = 1.0f + neg_exp(la);
    const float q = __builtin_amdgcn_rcpf(px * pa);
    g.gx = q * pa;
    g.ga = q * px;
    g.a0 = KNOWN ? a0 : __builtin_amdgcn_exp2f(k.k8 * g.ga);
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

// ------------------------------------------------- single-pass grouped scans
// One launch per direction on the grouped path (G <= RG_GROUP_MAX): a
// workgroup owns one group of G consecutive chunks (processing order) and 64
// lanes of channel pairs; wave w handles chunk w of the group.  Each wave
// reads its chunk's words once, forms the chunk's map (A, B) per channel
// for the group's LDS table, takes the state entering the group from the
// groups before it (rg_group_handoff) and runs the chunk from the state
// entering it.
constexpr int RG_GL = 64;  // lanes (channel pairs) per workgroup

// Hand-off words, per (group, lane), one per channel: the group's map for a
// group inside a segment, or the state leaving a segment's last group.  A
// map (A, B) is one word, B in the high half and -A in the low half: A is a
// product of retentions, never negative, so the low half of a published map
// has its sign bit set and a zeroed word reads as unpublished.  A state is
// a tagged word as in the complex scan ((1 << 32) | float bits, pub_store of
// common.hpp).  A 64-bit word is never torn, so no fence is needed.  Unlike
// the complex scan, the transition part of a group's map depends on every
// token's gate, so it travels with the affine part.
constexpr int RG_PUB_WORDS = 2;

__device__ __forceinline__ void pub_store_map(uint64_t* grp, int i, uint32_t Wb, uint32_t off, float a, float b) {
    __hip_atomic_store(pub_word(grp, i, Wb, off),
                       ((uint64_t)__float_as_uint(b) << 32) | (uint64_t)__float_as_uint(-a), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool map_ok(uint64_t w) { return ((uint32_t)w >> 31) != 0u; }

// The two words of an earlier group for this lane, once both are published
// (MAP: maps, else states; bounded wait, as wait_pair).  v = (A0, B0, A1, B1)
// for maps, (h0, h1, 0, 0) for states.
template <bool MAP>
__device__ __forceinline__ float4 wait_group(const uint64_t* grp, uint32_t Wb, uint32_t off, int polls) {
    const float nan = __builtin_nanf("");
    float4 v = make_float4(nan, nan, nan, nan);  // kept if the wait expires
    bool ok = false;
    for (int it = 0; it < polls; ++it) {
        if (!ok) {
            const uint32_t o = opaque_v(off);
            const uint64_t w0 = pub_load(grp, 0, Wb, o), w1 = pub_load(grp, 1, Wb, o);
            if (MAP ? (map_ok(w0) && map_ok(w1)) : (pub_ok(w0) && pub_ok(w1))) {
                v = MAP ? make_float4(-__uint_as_float((uint32_t)w0), __uint_as_float((uint32_t)(w0 >> 32)),
                                      -__uint_as_float((uint32_t)w1), __uint_as_float((uint32_t)(w1 >> 32)))
                        : make_float4(pub_val(w0), pub_val(w1), 0.f, 0.f);
                ok = true;
            }
        }
        if (__all(ok)) break;
        __builtin_amdgcn_s_sleep(1);
    }
    return v;
}

// The state entering group q (processing order) for this lane's two
// channels; the fixed-order segment chain of group_handoff (common.hpp)
// with real maps h -> A h + B per channel.  comp [G][64]: (A0, B0, A1, B1) of
// each of the group's chunks in processing order; look [G][64]: scratch;
// seed: the row's state before the first group (float2 per lane, NULL = 0);
// pub: the row's [NG][RG_PUB_WORDS][W] words; lw: the lane's word (clamped
// into the row, so that a lane past the row reads a published word).
__device__ __forceinline__ float2 rg_group_handoff(const float4* comp, float4* look, int G, int w, int lane, int q,
                                                   int NG, int W, int lw, bool active, const float2* seed,
                                                   uint64_t* pub, int polls) {
    const uint32_t Wb = (uint32_t)W * 8u, off = (uint32_t)lw * 8u;
    uint64_t* mine = pub + (size_t)q * RG_PUB_WORDS * W;  // wave-uniform
    const int nprev = q % G;
    const bool seg_last = nprev == G - 1 || q == NG - 1;
    if (w == 0 && active && q + 1 < NG && !seg_last) {
        // U_q = S_{G-1} o ... o S_0, composed in chunk order, published at once
        float a0 = 1.f, b0 = 0.f, a1 = 1.f, b1 = 0.f;
        for (int j = 0; j < G; ++j) {
            const float4 f = comp[j * RG_GL + lane];
            b0 = fmaf(f.x, b0, f.y);
            a0 *= f.x;
            b1 = fmaf(f.z, b1, f.w);
            a1 *= f.z;
        }
        pub_store_map(mine, 0, Wb, off, a0, b0);
        pub_store_map(mine, 1, Wb, off, a1, b1);
    }
    if (w < nprev) {
        look[w * RG_GL + lane] = wait_group<true>(pub + (size_t)(q - 1 - w) * RG_PUB_WORDS * W, Wb, off, polls);
    } else if (w == nprev) {
        float4 hs = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q - nprev > 0) {
            hs = wait_group<false>(pub + (size_t)(q - nprev - 1) * RG_PUB_WORDS * W, Wb, off, polls);
        } else if (seed) {
            const float2 h = seed[lw];
            hs = make_float4(h.x, h.y, 0.f, 0.f);
        }
        look[w * RG_GL + lane] = hs;
    }
    __syncthreads();
    if (w == 0) {
        const float4 hs = look[nprev * RG_GL + lane];
        float h0 = hs.x, h1 = hs.y;
        for (int v = nprev - 1; v >= 0; --v) {  // oldest first
            const float4 f = look[v * RG_GL + lane];
            h0 = fmaf(f.x, h0, f.y);
            h1 = fmaf(f.z, h1, f.w);
        }
        if (active && q + 1 < NG && seg_last) {
            float o0 = h0, o1 = h1;
            for (int j = 0; j < G; ++j) {
                const float4 f = comp[j * RG_GL + lane];
                o0 = fmaf(f.x, o0, f.y);
                o1 = fmaf(f.z, o1, f.w);
            }
            pub_store(mine, 0, Wb, off, o0);
            pub_store(mine, 1, Wb, off, o1);
        }
        look[lane] = make_float4(h0, h1, 0.f, 0.f);
    }
    __syncthreads();
    const float4 r = look[lane];
    return make_float2(r.x, r.y);
}

// Forward: every gate of the chunk is formed once; the chunk's retention
// and drive per token (a_t, x_t g^x_t m_t) stay in registers from the
// summary to the replay.
template <int K, bool F32>
__global__ __launch_bounds__(RG_GL * RG_GROUP_MAX) void rglru_gscan_kernel(
    int L, int W, int C, int G, const uint32_t* __restrict__ x, const uint32_t* __restrict__ lx,
    const uint32_t* __restrict__ la, const unsigned char* __restrict__ reset, const float* __restrict__ alpha,
    const float2* __restrict__ h0, uint64_t* __restrict__ pub, float2* __restrict__ entries, void* __restrict__ y,
    float2* __restrict__ h_final, int polls) {
    extern __shared__ float4 rg_lds[];  // comp [G][64], look [G][64]
    float4* const comp = rg_lds;
    float4* const look = rg_lds + G * RG_GL;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = blockIdx.y, b = blockIdx.z, NG = gridDim.y;
    const int c = q * G + w;
    const bool valid = c < C;  // wave-uniform
    const int lw0 = blockIdx.x * RG_GL + lane;
    const bool active = lw0 < W;
    const int lw = active ? lw0 : W - 1;
    const size_t tok0 = (size_t)b * L + (size_t)min(c, C - 1) * K;
    const int kc = valid ? min(K, L - c * K) : 0;
    const uint32_t rm = reset_mask<K>(reset, tok0, kc);
    const ChanConst k[2] = {chan_const(alpha[2 * lw]), chan_const(alpha[2 * lw + 1])};
    // the chunk's words (rows past its end read as 0 and are never used)
    uint32_t xs[K], lxs[K], las[K];
    {
        const ChunkRows rx(x + tok0 * W, kc, W), rl(lx + tok0 * W, kc, W), ra(la + tok0 * W, kc, W);
#pragma unroll
        for (int i = 0; i < K; ++i) {
            xs[i] = rx.load(i, lw);
            lxs[i] = rl.load(i, lw);
            las[i] = ra.load(i, lw);
        }
    }
    float av[K][2], bv[K][2];
    float A[2] = {1.f, 1.f}, Bs[2] = {0.f, 0.f};
    const int kq = opaque(kc);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (i < kq) {
            const bool rs = bit(rm, i);
            const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
            const float lxv[2] = {bf16_lo(lxs[i]), bf16_hi(lxs[i])};
            const float lav[2] = {bf16_lo(las[i]), bf16_hi(las[i])};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate g = gates(k[v], lxv[v], lav[v], rs);
                av[i][v] = g.a;
                bv[i][v] = xv[v] * g.gx * g.m;
                A[v] *= g.a;
                Bs[v] = fmaf(g.a, Bs[v], bv[i][v]);
            }
        }
    }
    comp[w * RG_GL + lane] = make_float4(A[0], Bs[0], A[1], Bs[1]);
    __syncthreads();
    const float2 hin = rg_group_handoff(comp, look, G, w, lane, q, NG, W, lw, active,
                                        h0 ? h0 + (size_t)b * W : nullptr, pub + (size_t)b * NG * RG_PUB_WORDS * W,
                                        polls);
    if (!valid) return;  // no barrier follows
    float h[2] = {hin.x, hin.y};
    for (int j = 0; j < w; ++j) {
        const float4 f = comp[j * RG_GL + lane];
        h[0] = fmaf(f.x, h[0], f.y);
        h[1] = fmaf(f.z, h[1], f.w);
    }
    if (active) entries[((size_t)b * C + c) * W + lw] = make_float2(h[0], h[1]);
    const ChunkOut yo(reinterpret_cast<char*>(y) + tok0 * (size_t)W * (F32 ? 8 : 4), K, W, F32 ? 8 : 4);
    const uint32_t yoff = (uint32_t)lw * (F32 ? 8u : 4u);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (i < kq) {
            h[0] = fmaf(av[i][0], h[0], bv[i][0]);
            h[1] = fmaf(av[i][1], h[1], bv[i][1]);
            if (active) {
                if (F32) yo.f32x2(i, yoff, h[0], h[1]);
                else yo.u32(i, yoff, pack_bf16x2(h[0], h[1]));
            }
        }
    }
    if (h_final && active && c == C - 1) h_final[(size_t)b * W + lw] = make_float2(h[0], h[1]);
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

// The forward recompute over H tokens whose words are held in registers,
// from the state h_in entering them: h_{t-1} of every token goes to the
// lane's LDS history.  SUMM: also the chunk's adjoint map carry_before =
// A carry_after + B with zero carry-in, formed in token order from the same
// retentions: A = prod a_t, B = sum_t (a_0 ... a_t) dy_t.
// KEEP: every token's retention a0 is kept in a0s for the reverse pass.
template <int H, bool FULL, bool SUMM, bool KEEP = false>
__device__ __forceinline__ void rg_bwd_forward(const ChanConst (&k)[2], int kq, uint32_t rm, const uint32_t (&xs)[H],
                                               const uint32_t (&lxs)[H], const uint32_t (&las)[H],
                                               const uint32_t (&gws)[H], const float (&h_in)[2], float2* hist,
                                               float (&A)[2], float (&Bv)[2], float (&a0s)[H][2]) {
    float h[2] = {h_in[0], h_in[1]};
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (FULL || i < kq) {
            const bool rs = bit(rm, i);
            const float xv[2] = {bf16_lo(xs[i]), bf16_hi(xs[i])};
            const float lxv[2] = {bf16_lo(lxs[i]), bf16_hi(lxs[i])};
            const float lav[2] = {bf16_lo(las[i]), bf16_hi(las[i])};
            const float gv[2] = {bf16_lo(gws[i]), bf16_hi(gws[i])};
            hist[i * 64] = make_float2(h[0], h[1]);
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const Gate g = gates(k[v], lxv[v], lav[v], rs);
                if (KEEP) a0s[i][v] = g.a0;
                h[v] = fmaf(g.a, h[v], xv[v] * g.gx * g.m);
                if (SUMM) {
                    A[v] *= g.a;
                    Bv[v] = fmaf(A[v], gv[v], Bv[v]);
                }
            }
        }
    }
}

// The adjoint over H tokens in reverse, from the cotangent `carry` arriving
// after them, with h_{t-1} from the LDS history; `active` = the lane's
// outputs are stored; KEEP: the retentions come from the forward pass.
template <int H, bool F32, bool FULL, bool KEEP = false>
__device__ __forceinline__ void rg_bwd_reverse(const RgIn& in, const ChanConst (&k)[2], const RgBwdOut& o,
                                               size_t tok0, int lw, int kq, uint32_t rm, bool active,
                                               const uint32_t (&xs)[H], const uint32_t (&lxs)[H],
                                               const uint32_t (&las)[H], const uint32_t (&gws)[H],
                                               float (&carry)[2], float (&acc)[2], const float2* hist,
                                               const float (&a0s)[H][2]) {
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
                const Gate gt = gates<KEEP>(k[v], lxv[v], lav[v], rs, a0s[i][v]);
                const float g = gv[v] + carry[v];
                const float xg = xv[v] * gt.gx;
                // dx = g g^x m; dl^x = g m x g^x (1 - g^x), with x g^x (1 - g^x)
                // = xg - xg g^x
                const float gm = g * gt.m;
                ox[v] = gm * gt.gx;
                olx[v] = gm * fmaf(-xg, gt.gx, xg);
                // d h / d a = h_{t-1} + x g^x dm/da, dm/da = -a / sqrt(u) (capped);
                // zero at a segment start, where a and m are constants
                const float dm_da = -gt.a0 * fminf(gt.r, RG_RSQ_CAP);
                const float abar = rs ? 0.0f : g * fmaf(xg, dm_da, hpv[v]);
                // d a / d l^a = a (-8 sp) g^a (1 - g^a); d a / d alpha = a g^a (-8 sigmoid(alpha))
                const float ag = abar * (gt.a0 * gt.ga);
                const float ags = ag * k[v].sp8;
                ola[v] = fmaf(-ags, gt.ga, ags);
                acc[v] += ag;
                carry[v] = gt.a * g;
            }
            const size_t row = (tok0 + i) * (size_t)in.W;
            if (F32 && active) {
                out_f32x2(reinterpret_cast<float2*>(o.dx) + row + lw, ox[0], ox[1]);
                out_f32x2(reinterpret_cast<float2*>(o.dlx) + row + lw, olx[0], olx[1]);
                out_f32x2(reinterpret_cast<float2*>(o.dla) + row + lw, ola[0], ola[1]);
            } else if (active) {
                out_u32(reinterpret_cast<uint32_t*>(o.dx) + row + lw, pack_bf16x2(ox[0], ox[1]));
                out_u32(reinterpret_cast<uint32_t*>(o.dlx) + row + lw, pack_bf16x2(olx[0], olx[1]));
                out_u32(reinterpret_cast<uint32_t*>(o.dla) + row + lw, pack_bf16x2(ola[0], ola[1]));
            }
        }
    }
}


template <int H, bool F32, bool FULL>
__device__ __forceinline__ void rg_bwd_words(const RgIn& in, const ChanConst (&k)[2], const RgBwdOut& o,
                                             size_t tok0, int lw, int kq, uint32_t rm, const uint32_t (&xs)[H],
                                             const uint32_t (&lxs)[H], const uint32_t (&las)[H],
                                             const uint32_t (&gws)[H], const float (&h_in)[2], float (&carry)[2],
                                             float (&acc)[2], float2* hist) {
    float A[2], Bv[2], a0s[H][2];
    rg_bwd_forward<H, FULL, false>(k, kq, rm, xs, lxs, las, gws, h_in, hist, A, Bv, a0s);
    asm volatile("" ::: "memory");  // read the history back from LDS, not from registers
    rg_bwd_reverse<H, F32, FULL>(in, k, o, tok0, lw, kq, rm, true, xs, lxs, las, gws, carry, acc, hist, a0s);
}

template <int H, bool F32, bool FULL>
__device__ __forceinline__ void rg_bwd_sub(const RgIn& in, const ChanConst (&k)[2], const RgBwdOut& o,
                                           size_t tok0, int lw, int kq, uint32_t rm,
                                           const float (&h_in)[2], float (&carry)[2], float (&acc)[2],
                                           float2* hist) {
    uint32_t xs[H], lxs[H], las[H], gws[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
        if (FULL || i < kq) {
            xs[i] = word(in.x, tok0, i, in.W, lw);
            lxs[i] = word(in.lx, tok0, i, in.W, lw);
            las[i] = word(in.la, tok0, i, in.W, lw);
            gws[i] = word(o.dy, tok0, i, in.W, lw);
        }
    }
    rg_bwd_words<H, F32, FULL>(in, k, o, tok0, lw, kq, rm, xs, lxs, las, gws, h_in, carry, acc, hist);
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

// The single-pass backward keeps each token's retention from the forward
// recompute to the reverse pass (one special function fewer per channel
// and token in the reverse pass, 32 more registers).
#ifndef LRS_RG_GB_KEEP
#define LRS_RG_GB_KEEP 1
#endif
constexpr bool RG_GB_KEEP = LRS_RG_GB_KEEP != 0;

// Single-pass backward: wave w of group q takes chunk C - 1 - (q G + w)
// (processing order runs backward in time).  Its words (x, l^x, l^a, dy) are
// read once.  Before the hand-off, the forward recompute runs from the
// chunk's saved entry state (h_{t-1} into the lane's LDS history) and, from
// the same retentions, forms the chunk's adjoint map for the group's table;
// the carry arriving after the chunk then comes from the hand-off and the
// group's later chunks, and the reverse pass (gates evaluated again) runs
// from it.  The alpha partials of the group's chunks are added in
// processing order into one row per group.
template <int K, bool F32>
__global__ __launch_bounds__(RG_GL * RG_GROUP_MAX) void rglru_gbscan_kernel(
    int L, int W, int C, int G, const uint32_t* __restrict__ x, const uint32_t* __restrict__ lx,
    const uint32_t* __restrict__ la, const unsigned char* __restrict__ reset, const float* __restrict__ alpha,
    const float2* __restrict__ entries, const float2* __restrict__ dh_final, uint64_t* __restrict__ pub,
    const uint32_t* __restrict__ dy, void* __restrict__ dx, void* __restrict__ dlx, void* __restrict__ dla,
    float2* __restrict__ dh0, float2* __restrict__ alpha_part, int polls) {
    extern __shared__ float4 rg_lds[];  // comp [G][64], look [G][64], hist [G][K][64] float2
    float4* const comp = rg_lds;
    float4* const look = rg_lds + G * RG_GL;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float2* const hist = reinterpret_cast<float2*>(rg_lds + 2 * G * RG_GL) + (size_t)w * K * RG_GL + lane;
    const int q = blockIdx.y, b = blockIdx.z, NG = gridDim.y;
    const int pc = q * G + w;
    const bool valid = pc < C;  // wave-uniform
    const int c = C - 1 - min(pc, C - 1);
    const int lw0 = blockIdx.x * RG_GL + lane;
    const bool active = lw0 < W;
    const int lw = active ? lw0 : W - 1;
    const size_t tok0 = (size_t)b * L + (size_t)c * K;
    const int kc = valid ? min(K, L - c * K) : 0;
    const uint32_t rm = reset_mask<K>(reset, tok0, kc);
    const ChanConst k[2] = {chan_const(alpha[2 * lw]), chan_const(alpha[2 * lw + 1])};
    const float2 e = entries[((size_t)b * C + c) * W + lw];
    uint32_t xs[K], lxs[K], las[K], gws[K];
    {
        // the pass's only read of these words, and the step's last: the
        // non-temporal hint keeps them out of the memory-side cache
        const ChunkRows rx(x + tok0 * W, kc, W), rl(lx + tok0 * W, kc, W), ra(la + tok0 * W, kc, W),
            rg(dy + tok0 * W, kc, W);
#pragma unroll
        for (int i = 0; i < K; ++i) {
            xs[i] = rx.load_nt(i, lw);
            lxs[i] = rl.load_nt(i, lw);
            las[i] = ra.load_nt(i, lw);
            gws[i] = rg.load_nt(i, lw);
        }
    }
    const int kq = opaque(kc);
    float A[2] = {1.f, 1.f}, Bv[2] = {0.f, 0.f}, a0s[K][2];
    {
        const float h_in[2] = {e.x, e.y};
        rg_bwd_forward<K, false, true, RG_GB_KEEP>(k, kq, rm, xs, lxs, las, gws, h_in, hist, A, Bv, a0s);
    }
    comp[w * RG_GL + lane] = make_float4(A[0], Bv[0], A[1], Bv[1]);
    __syncthreads();
    const float2 cin = rg_group_handoff(comp, look, G, w, lane, q, NG, W, lw, active,
                                        dh_final ? dh_final + (size_t)b * W : nullptr,
                                        pub + (size_t)b * NG * RG_PUB_WORDS * W, polls);
    float carry[2] = {cin.x, cin.y};
    for (int j = 0; j < w; ++j) {
        const float4 f = comp[j * RG_GL + lane];
        carry[0] = fmaf(f.x, carry[0], f.y);
        carry[1] = fmaf(f.z, carry[1], f.w);
    }
    float acc[2] = {0.f, 0.f};
    if (valid) {
        const RgIn in{L, W, x, lx, la, reset};
        const RgBwdOut o{dy, dx, dlx, dla};
        rg_bwd_reverse<K, F32, false, RG_GB_KEEP>(in, k, o, tok0, lw, kq, rm, active, xs, lxs, las, gws, carry,
                                                  acc, hist, a0s);
        if (dh0 && active && c == 0) dh0[(size_t)b * W + lw] = make_float2(carry[0], carry[1]);
    }
    // the alpha partials of the group's chunks, in processing order, through
    // each wave's own history slots (free once its reverse pass is done)
    hist[0] = make_float2(acc[0] * k[0].dsp8, acc[1] * k[1].dsp8);
    __syncthreads();
    if (w == 0 && active) {
        const float2* part = reinterpret_cast<const float2*>(rg_lds + 2 * G * RG_GL) + lane;
        const int n = min(G, C - q * G);
        float s0 = 0.f, s1 = 0.f;
        for (int j = 0; j < n; ++j) {
            const float2 v = part[(size_t)j * K * RG_GL];
            s0 += v.x;
            s1 += v.y;
        }
        alpha_part[((size_t)b * NG + q) * W + lw] = make_float2(s0, s1);
    }
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

hipError_t launch_rglru_alpha_reduce(const RglruParams& p, int rows, const float* alpha_part, float* dalpha,
                                     hipStream_t s) {
    LRS_LAUNCH(K_RGLRU_ALPHA, rglru_alpha_kernel, dim3((unsigned)ceil_div(p.D, AR_COLS)), dim3(AR_THREADS), 0, s,
               rows, p.D, alpha_part, dalpha);
    return hipGetLastError();
}

bool rglru_fused(const Chunking& ch) { return ch.K == 16 && ch.G <= RG_GROUP_MAX; }

size_t rglru_pub_bytes(const Chunking& ch, int D) {
    return (size_t)ch.B * ch.NG * RG_PUB_WORDS * (size_t)(D / 2) * sizeof(uint64_t);
}

hipError_t launch_rglru_gscan(const RglruParams& p, const Chunking& ch, void* pub, size_t pub_bytes,
                              float* entries, void* y, int y_f32, float* h_final, hipStream_t s) {
    if (ch.NG > 1) {
        const hipError_t e = launch_clear_words(pub, pub_bytes, s);
        if (e != hipSuccess) return e;
    }
    const int W = p.D / 2;
    const dim3 grid((unsigned)ceil_div(W, RG_GL), ch.NG, ch.B);
    const dim3 block(RG_GL * ch.G);
    const size_t lds = (size_t)2 * ch.G * RG_GL * sizeof(float4);
#define RG_GSCAN(FF)                                                                                           \
    LRS_LAUNCH(K_RGLRU_FWD_SCAN, (rglru_gscan_kernel<16, FF>), grid, block, lds, s, p.L, W, ch.C, ch.G,          \
               (const uint32_t*)p.x, (const uint32_t*)p.lx, (const uint32_t*)p.la, p.reset, p.alpha,            \
               (const float2*)p.h0, (uint64_t*)pub, (float2*)entries, y, (float2*)h_final, handoff_poll_limit())
    if (y_f32) RG_GSCAN(true);
    else RG_GSCAN(false);
#undef RG_GSCAN
    return hipGetLastError();
}

hipError_t launch_rglru_gbscan(const RglruParams& p, const Chunking& ch, const float* entries,
                               const float* dh_final, void* pub, size_t pub_bytes, const void* dy, void* dx,
                               void* dlx, void* dla, int g_f32, float* dh0, float* alpha_part, hipStream_t s) {
    if (ch.NG > 1) {
        const hipError_t e = launch_clear_words(pub, pub_bytes, s);
        if (e != hipSuccess) return e;
    }
    const int W = p.D / 2;
    const dim3 grid((unsigned)ceil_div(W, RG_GL), ch.NG, ch.B);
    const dim3 block(RG_GL * ch.G);
    // the map table, the hand-off scratch and the h histories
    const size_t lds = (size_t)2 * ch.G * RG_GL * sizeof(float4) + (size_t)ch.G * 16 * RG_GL * sizeof(float2);
#define RG_GBSCAN(FF)                                                                                          \
    LRS_LAUNCH(K_RGLRU_BWD_SCAN, (rglru_gbscan_kernel<16, FF>), grid, block, lds, s, p.L, W, ch.C, ch.G,         \
               (const uint32_t*)p.x, (const uint32_t*)p.lx, (const uint32_t*)p.la, p.reset, p.alpha,            \
               (const float2*)entries, (const float2*)dh_final, (uint64_t*)pub, (const uint32_t*)dy, dx, dlx,   \
               dla, (float2*)dh0, (float2*)alpha_part, handoff_poll_limit())
    if (g_f32) RG_GBSCAN(true);
    else RG_GBSCAN(false);
#undef RG_GBSCAN
    return hipGetLastError();
}

}  // namespace lrs
