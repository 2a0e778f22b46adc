// samu_fwd.hip -- SAMU forward kernels for gfx950 and the reverse chunk
// summary of the backward pass.
//
// Page 'SAMU 与 RG-LRU 的 H800 训练性能对比', section 05:
//   controller   x~ = [x_sel; 1], w^ = w/||w||, p = tanh(x~.w^_phi),
//                r = tanh(x~.w^_r), q = r/(1+r^2), d = tanh(a_phi)/sqrt(M) p,
//                c = tanh(a_r)/sqrt(M) q, then E = e^c, C = cos d, S = sin d once
//                per token;
//   transition   lambda_{t,m} built in registers from (E, C, S) and (nu_m, theta_m),
//                never written to memory;
//   recurrence   z_t = lambda_t z_{t-1} + b_t; K consecutive steps compose into
//                one affine summary S_c (the right operand runs first);
//   replay       rerun K steps from the chunk's entry state, writing y = z.
// The backward's reverse summary (same section, 'backward' list, first item)
// composes carry -> conj(lambda_t) (dy_t + carry) over a chunk from its last
// token to its first.
//
// Layout: lanes run over modes (VM consecutive modes per lane, so one BF16
// complex drive word per mode and one 4*VM-byte load per token); a workgroup
// owns one chunk of one batch row and a slice of the modes, so every wave
// streams contiguous rows of the [B, L, M, 2] tensors.  Token controls are
// wave-uniform and arrive through the scalar cache.
#include "common.hpp"

namespace lrs {
namespace {

// ------------------------------------------------------------------ K1 ---
constexpr int CTL_THREADS = 256;        // 4 waves
constexpr int CTL_TOK_PER_PASS = 4;     // tokens reduced together per wave
constexpr int CTL_PASSES = 4;
constexpr int CTL_TOK_PER_BLOCK = 4 * CTL_TOK_PER_PASS * CTL_PASSES;

__global__ __launch_bounds__(CTL_THREADS) void samu_controller_kernel(
    int BL, int D, int M, const uint4* __restrict__ x_sel, const float* __restrict__ w_phi,
    const float* __restrict__ w_r, const float* __restrict__ a_phi,
    const float* __restrict__ a_r, float* __restrict__ p_out, float* __restrict__ r_out,
    TokenCtl* __restrict__ ctl) {
    __shared__ float red[2][CTL_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // direction norms over all D+1 entries
    float sp = 0.f, sr = 0.f;
    for (int j = tid; j <= D; j += CTL_THREADS) {
        sp = fmaf(w_phi[j], w_phi[j], sp);
        sr = fmaf(w_r[j], w_r[j], sr);
    }
    sp = wave_sum(sp);
    sr = wave_sum(sr);
    if (lane == 0) { red[0][wave] = sp; red[1][wave] = sr; }
    __syncthreads();
    float np = 0.f, nr = 0.f;
#pragma unroll
    for (int i = 0; i < CTL_THREADS / 64; ++i) { np += red[0][i]; nr += red[1][i]; }
    const float inv_phi = 1.0f / sqrtf(np), inv_r = 1.0f / sqrtf(nr);
    const float amp_phi = tanhf(a_phi[0]) / sqrtf((float)M);
    const float amp_r = tanhf(a_r[0]) / sqrtf((float)M);
    const float bias_phi = w_phi[D], bias_r = w_r[D];

    const int D8 = D >> 3;  // 16-byte words per row
    for (int pass = 0; pass < CTL_PASSES; ++pass) {
        const int tok0 = blockIdx.x * CTL_TOK_PER_BLOCK + (wave * CTL_PASSES + pass) * CTL_TOK_PER_PASS;
        float ap[CTL_TOK_PER_PASS], ar[CTL_TOK_PER_PASS];
#pragma unroll
        for (int q = 0; q < CTL_TOK_PER_PASS; ++q) { ap[q] = 0.f; ar[q] = 0.f; }
        for (int j = lane; j < D8; j += 64) {
            const float4 wp0 = reinterpret_cast<const float4*>(w_phi)[2 * j];
            const float4 wp1 = reinterpret_cast<const float4*>(w_phi)[2 * j + 1];
            const float4 wr0 = reinterpret_cast<const float4*>(w_r)[2 * j];
            const float4 wr1 = reinterpret_cast<const float4*>(w_r)[2 * j + 1];
            const float wp[8] = {wp0.x, wp0.y, wp0.z, wp0.w, wp1.x, wp1.y, wp1.z, wp1.w};
            const float wr[8] = {wr0.x, wr0.y, wr0.z, wr0.w, wr1.x, wr1.y, wr1.z, wr1.w};
#pragma unroll
            for (int q = 0; q < CTL_TOK_PER_PASS; ++q) {
                const int tok = tok0 + q;
                if (tok < BL) {
                    const uint4 xv = x_sel[(size_t)tok * D8 + j];
                    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x0 = bf16_lo(xw[e]), x1 = bf16_hi(xw[e]);
                        ap[q] = fmaf(x0, wp[2 * e], ap[q]);
                        ap[q] = fmaf(x1, wp[2 * e + 1], ap[q]);
                        ar[q] = fmaf(x0, wr[2 * e], ar[q]);
                        ar[q] = fmaf(x1, wr[2 * e + 1], ar[q]);
                    }
                }
            }
        }
        float up = 0.f, ur = 0.f;
#pragma unroll
        for (int q = 0; q < CTL_TOK_PER_PASS; ++q) {
            const float sp_q = wave_sum(ap[q]), sr_q = wave_sum(ar[q]);
            if (lane == q) { up = sp_q; ur = sr_q; }
        }
        const int tok = tok0 + lane;
        if (lane < CTL_TOK_PER_PASS && tok < BL) {
            const float p = tanhf((up + bias_phi) * inv_phi);
            const float r = tanhf((ur + bias_r) * inv_r);
            const float q = r / (1.0f + r * r);
            const float d = amp_phi * p, c = amp_r * q;
            p_out[tok] = p;
            r_out[tok] = r;
            float sd, cd;
            sincosf(d, &sd, &cd);
            TokenCtl t;
            t.E = expf(c);
            t.C = cd;
            t.S = sd;
            t.pad = 0.f;
            ctl[tok] = t;
        }
    }
}

// ---------------------------------------------------------- K2 / K5 ---
template <int VM> struct Words;
template <> struct Words<1> {
    uint32_t w[1];
    __device__ void load(const uint32_t* p) { w[0] = *p; }
};
template <> struct Words<2> {
    uint32_t w[2];
    __device__ void load(const uint32_t* p) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x; w[1] = v.y;
    }
};
template <> struct Words<4> {
    uint32_t w[4];
    __device__ void load(const uint32_t* p) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
};

constexpr int SUM_VM = 4;

// One step of the forward summary (REV = false) or of the reverse conjugate
// summary (REV = true) for the VM modes of this lane.
template <int VM, bool REV>
__device__ __forceinline__ void summary_step(const ModeConst (&k)[VM], cf (&A)[VM], cf (&Bv)[VM],
                                             const TokenCtl& tc, const Words<VM>& dw) {
#pragma unroll
    for (int v = 0; v < VM; ++v) {
        const cf lam = mode_lambda(k[v], tc.E, tc.C, tc.S);
        const cf x = {bf16_lo(dw.w[v]), bf16_hi(dw.w[v])};
        if (!REV) {
            // (lam, x) o (A, B) = (lam A, lam B + x)
            A[v] = cmul(lam, A[v]);
            Bv[v] = cfma(lam, Bv[v], x);
        } else {
            // carry -> conj(lam) (x + carry)
            A[v] = cmulc(lam, A[v]);
            Bv[v] = cmulc(lam, {Bv[v].re + x.re, Bv[v].im + x.im});
        }
    }
}

template <int VM, int K, bool REV>
__global__ __launch_bounds__(256) void samu_summary_kernel(
    int L, int M, int C, const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
    const float* __restrict__ nu, const float* __restrict__ theta, float* __restrict__ summ) {
    const int m0 = (blockIdx.x * blockDim.x + threadIdx.x) * VM;
    const int c = blockIdx.y, b = blockIdx.z;
    if (m0 >= M) return;
    ModeConst k[VM];
#pragma unroll
    for (int v = 0; v < VM; ++v) k[v] = mode_const(nu[m0 + v], theta[m0 + v]);
    cf A[VM], Bv[VM];
#pragma unroll
    for (int v = 0; v < VM; ++v) { A[v] = {1.f, 0.f}; Bv[v] = {0.f, 0.f}; }

    const int s = c * K;
    const int kc = min(K, L - s);
    const TokenCtl* tc = ctl + (size_t)b * L + s;
    const uint32_t* dp = drive + ((size_t)b * L + s) * M + m0;
    if (kc == K) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int i = REV ? K - 1 - j : j;
            Words<VM> w;
            w.load(dp + (size_t)i * M);
            summary_step<VM, REV>(k, A, Bv, tc[i], w);
        }
    } else {
        for (int j = 0; j < kc; ++j) {
            const int i = REV ? kc - 1 - j : j;
            Words<VM> w;
            w.load(dp + (size_t)i * M);
            summary_step<VM, REV>(k, A, Bv, tc[i], w);
        }
    }
    float4* out = reinterpret_cast<float4*>(summ) + ((size_t)b * C + c) * M + m0;
#pragma unroll
    for (int v = 0; v < VM; ++v) out[v] = make_float4(A[v].re, A[v].im, Bv[v].re, Bv[v].im);
}

// ------------------------------------------------------------------ K4 ---
constexpr int REP_VM = 4;

template <int VM, bool F32>
__device__ __forceinline__ void store_states(void* y, size_t idx, const cf (&z)[VM]) {
    if (F32) {
        float2* o = reinterpret_cast<float2*>(y) + idx;
        if (VM == 4) {
            reinterpret_cast<float4*>(o)[0] = make_float4(z[0].re, z[0].im, z[1].re, z[1].im);
            reinterpret_cast<float4*>(o)[1] = make_float4(z[2].re, z[2].im, z[3].re, z[3].im);
        } else {
#pragma unroll
            for (int v = 0; v < VM; ++v) o[v] = make_float2(z[v].re, z[v].im);
        }
    } else {
        uint32_t* o = reinterpret_cast<uint32_t*>(y) + idx;
        if (VM == 4) {
            *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(z[0].re, z[0].im), pack_bf16x2(z[1].re, z[1].im),
                                                      pack_bf16x2(z[2].re, z[2].im), pack_bf16x2(z[3].re, z[3].im));
        } else {
#pragma unroll
            for (int v = 0; v < VM; ++v) o[v] = pack_bf16x2(z[v].re, z[v].im);
        }
    }
}

template <int VM, int K, bool F32>
__global__ __launch_bounds__(256) void samu_replay_kernel(
    int L, int M, int C, const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
    const float* __restrict__ nu, const float* __restrict__ theta,
    const float* __restrict__ entries, void* __restrict__ y, float* __restrict__ z_final) {
    const int m0 = (blockIdx.x * blockDim.x + threadIdx.x) * VM;
    const int c = blockIdx.y, b = blockIdx.z;
    if (m0 >= M) return;
    ModeConst k[VM];
    cf z[VM];
    const float2* ent = reinterpret_cast<const float2*>(entries) + ((size_t)b * C + c) * M + m0;
#pragma unroll
    for (int v = 0; v < VM; ++v) {
        k[v] = mode_const(nu[m0 + v], theta[m0 + v]);
        const float2 e = ent[v];
        z[v] = {e.x, e.y};
    }
    const int s = c * K;
    const int kc = min(K, L - s);
    const TokenCtl* tc = ctl + (size_t)b * L + s;
    const size_t row0 = ((size_t)b * L + s) * M + m0;
    auto step = [&](int i) {
        Words<VM> w;
        w.load(drive + row0 + (size_t)i * M);
        const TokenCtl t = tc[i];
#pragma unroll
        for (int v = 0; v < VM; ++v) {
            const cf lam = mode_lambda(k[v], t.E, t.C, t.S);
            z[v] = cfma(lam, z[v], {bf16_lo(w.w[v]), bf16_hi(w.w[v])});
        }
        store_states<VM, F32>(y, row0 + (size_t)i * M, z);
    };
    if (kc == K) {
#pragma unroll
        for (int i = 0; i < K; ++i) step(i);
    } else {
        for (int i = 0; i < kc; ++i) step(i);
    }
    if (z_final && c == C - 1) {
        float2* zf = reinterpret_cast<float2*>(z_final) + (size_t)b * M + m0;
#pragma unroll
        for (int v = 0; v < VM; ++v) zf[v] = make_float2(z[v].re, z[v].im);
    }
}

inline int mode_block(int M, int VM) {
    const int lanes = (int)ceil_div(M, VM);
    return lanes >= 256 ? 256 : (int)ceil_div(lanes, 64) * 64;
}

}  // namespace

hipError_t launch_samu_controller(const SamuParams& p, float* p_out, float* r_out, float* ctl,
                                  hipStream_t s) {
    const int BL = p.B * p.L;
    const int grid = (int)ceil_div(BL, CTL_TOK_PER_BLOCK);
    LRS_LAUNCH(K_SAMU_CONTROLLER, samu_controller_kernel, dim3(grid), dim3(CTL_THREADS), 0, s,
               BL, p.D, p.M, (const uint4*)p.x_sel, p.w_phi, p.w_r, p.a_phi, p.a_r, p_out, r_out,
               (TokenCtl*)ctl);
    return hipGetLastError();
}

hipError_t launch_samu_summary(const SamuParams& p, const Chunking& ch, const float* ctl,
                               const void* drive, bool reverse, float* summ, hipStream_t s) {
    const int blk = mode_block(p.M, SUM_VM);
    const dim3 grid((unsigned)ceil_div(ceil_div(p.M, SUM_VM), blk), ch.C, ch.B);
    const int id = reverse ? K_SAMU_REV_SUMMARY : K_SAMU_SUMMARY;
#define SUMMARY_CASE(KK, RR)                                                                        \
    LRS_LAUNCH(id, (samu_summary_kernel<SUM_VM, KK, RR>), grid, dim3(blk), 0, s, p.L, p.M, ch.C, \
               (const TokenCtl*)ctl, (const uint32_t*)drive, p.nu, p.theta, summ)
    if (ch.K == 32) {
        if (reverse) SUMMARY_CASE(32, true); else SUMMARY_CASE(32, false);
    } else {
        if (reverse) SUMMARY_CASE(16, true); else SUMMARY_CASE(16, false);
    }
#undef SUMMARY_CASE
    return hipGetLastError();
}

hipError_t launch_samu_replay(const SamuParams& p, const Chunking& ch, const float* ctl,
                              const float* entries, void* y, int y_f32, float* z_final,
                              hipStream_t s) {
    const int blk = mode_block(p.M, REP_VM);
    const dim3 grid((unsigned)ceil_div(ceil_div(p.M, REP_VM), blk), ch.C, ch.B);
#define REPLAY_CASE(KK, FF)                                                                       \
    LRS_LAUNCH(K_SAMU_REPLAY, (samu_replay_kernel<REP_VM, KK, FF>), grid, dim3(blk), 0, s, p.L, \
               p.M, ch.C, (const TokenCtl*)ctl, (const uint32_t*)p.b, p.nu, p.theta, entries, y, \
               z_final)
    if (ch.K == 32) {
        if (y_f32) REPLAY_CASE(32, true); else REPLAY_CASE(32, false);
    } else {
        if (y_f32) REPLAY_CASE(16, true); else REPLAY_CASE(16, false);
    }
#undef REPLAY_CASE
    return hipGetLastError();
}

}  // namespace lrs
