// samu_bwd.hip -- SAMU backward kernels for gfx950.
//
// Page 'SAMU 与 RG-LRU 的 H800 训练性能对比', section 05 ('backward' list and
// the z-bar, c-bar/d-bar and p-bar/r-bar displays), and page 'SAMU
// strengthened-baseline H800 report', 'Reverse complex backward':
//   * the state cotangent runs through conj(lambda) in reversed time,
//     z-bar_{t-1} += conj(lambda_t) z-bar_t and b-bar_t = z-bar_t;
//   * a replay regenerates lambda in registers and yields the drive, nu and
//     theta gradients without any stored transition history;
//   * every mode tile emits two controller partial sums per token, and a
//     deterministic FP32 second stage reduces [B, L, N_tiles, 2] to [B, L, 2];
//   * the controller backward uses the saved p, r:
//     p-bar = d-bar tanh(a_phi)/sqrt(M), r-bar = c-bar tanh(a_r)/sqrt(M)
//     (1 - r^2)/(1 + r^2)^2, then tanh', the direction normalization and
//     the amplitude chain rule.
// With gamma = conj(lambda_t) g_t conj(z_{t-1}) = g_t conj(lambda_t z_{t-1}):
//   d nu_m = -sum E_t Re gamma,  d theta_m = sum Im gamma,
//   c-bar_t = -E_t sum_m nu_m Re gamma,  d-bar_t = sum_m Im gamma.
// No atomics anywhere: every sum has a fixed order, so results are bitwise
// reproducible run to run.
#include "common.hpp"

namespace lrs {
namespace {

// ------------------------------------------------------------------ K7 ---
// One lane per mode, one workgroup per (chunk, 128 modes).  The forward
// recompute keeps lambda_t and w_t = lambda_t z_{t-1} of the chunk in
// registers; the reverse pass consumes them.  The per-token partial sums of a
// wave are reduced through a padded LDS transpose (conflict-free both ways).
constexpr int BWD_THREADS = 128;
constexpr int BWD_PAD = 65;

template <int K, bool F32>
__global__ __launch_bounds__(BWD_THREADS) void samu_bwd_replay_kernel(
    int L, int M, int C, int n_tiles, const TokenCtl* __restrict__ ctl,
    const uint32_t* __restrict__ drive, const float* __restrict__ nu,
    const float* __restrict__ theta, const float2* __restrict__ entries,
    const float2* __restrict__ carry_in, const uint32_t* __restrict__ dy, void* __restrict__ db,
    float2* __restrict__ dz0, float* __restrict__ tok_part, float2* __restrict__ mode_part) {
    static_assert(2 * K <= 64, "one transposed row per lane");
    __shared__ float lds[BWD_THREADS / 64][64 * BWD_PAD];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = blockIdx.x * BWD_THREADS + threadIdx.x;
    const int c = blockIdx.y, b = blockIdx.z;
    const bool active = m < M;
    const int mm = active ? m : M - 1;
    const ModeConst k = mode_const(nu[mm], theta[mm]);
    const float num = nu[mm];

    const int s = c * K;
    const int kc = min(K, L - s);
    const TokenCtl* tc = ctl + (size_t)b * L + s;
    const size_t row0 = ((size_t)b * L + s) * M + mm;
    const size_t cidx = ((size_t)b * C + c) * M + mm;

    // forward recompute of the chunk from its saved entry state
    cf lam[K], wz[K];
    {
        const float2 e = entries[cidx];
        cf z = {e.x, e.y};
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (i < kc) {
                const TokenCtl t = tc[i];
                const uint32_t bw = drive[row0 + (size_t)i * M];
                lam[i] = mode_lambda(k, t.E, t.C, t.S);
                wz[i] = cmul(lam[i], z);
                z = {wz[i].re + bf16_lo(bw), wz[i].im + bf16_hi(bw)};
            }
        }
    }

    // reverse adjoint over the chunk
    const float2 ci = carry_in[cidx];
    cf carry = {ci.x, ci.y};
    float acc_nu = 0.f, acc_th = 0.f;
    float* row = &lds[wave][lane * BWD_PAD];
#pragma unroll
    for (int i = K - 1; i >= 0; --i) {
        float pr = 0.f, pi = 0.f;
        if (i < kc) {
            const float E = tc[i].E;
            const uint32_t gw = dy[row0 + (size_t)i * M];
            const cf g = {bf16_lo(gw) + carry.re, bf16_hi(gw) + carry.im};
            if (active) {
                if (F32) reinterpret_cast<float2*>(db)[row0 + (size_t)i * M] = make_float2(g.re, g.im);
                else reinterpret_cast<uint32_t*>(db)[row0 + (size_t)i * M] = pack_bf16x2(g.re, g.im);
            }
            // gamma = g conj(w)
            const float gre = fmaf(g.re, wz[i].re, g.im * wz[i].im);
            const float gim = fmaf(g.im, wz[i].re, -g.re * wz[i].im);
            acc_nu = fmaf(E, gre, acc_nu);
            acc_th += gim;
            pr = num * gre;
            pi = gim;
            carry = cmulc(lam[i], g);
        }
        if (!active) { pr = 0.f; pi = 0.f; }
        row[2 * i] = pr;
        row[2 * i + 1] = pi;
    }
    if (active) {
        mode_part[cidx] = make_float2(-acc_nu, acc_th);
        if (dz0 && c == 0) dz0[(size_t)b * M + mm] = make_float2(carry.re, carry.im);
    }
    __syncthreads();
    // lane j sums column j (token j/2, component j%2) over the 64 modes of the wave
    if (lane < 2 * kc) {
        float acc = 0.f;
        const float* col = &lds[wave][lane];
#pragma unroll 16
        for (int r = 0; r < 64; ++r) acc += col[r * BWD_PAD];
        const int t = lane >> 1;
        if ((lane & 1) == 0) acc *= -tc[t].E;
        const int tile = blockIdx.x * (BWD_THREADS / 64) + wave;
        if (tile < n_tiles)
            tok_part[(((size_t)b * n_tiles + tile) * L + s) * 2 + lane] = acc;
    }
}

// ------------------------------------------------------------------ K9 ---
// One workgroup per block of CTL_TB tokens; each thread owns 8 selector
// columns.  The first stage of the shared-control reduction (over mode tiles)
// happens here in fixed tile order, then p-bar, r-bar and the per-token u-bar
// follow; dx_sel = u-bar_phi w^_phi + u-bar_r w^_r, and the block's partial
// sums of u-bar * x~ (direction gradients) plus sum d-bar p, sum c-bar q are
// written for the final deterministic reduction.
constexpr int CTL_TB = 64;

template <bool F32>
__global__ __launch_bounds__(512) void samu_ctl_bwd_kernel(
    int B, int L, int D, int M, int n_tiles, const uint4* __restrict__ x_sel,
    const float* __restrict__ w_phi, const float* __restrict__ w_r,
    const float* __restrict__ a_phi, const float* __restrict__ a_r,
    const float* __restrict__ p_sv, const float* __restrict__ r_sv,
    const float* __restrict__ tok_part, void* __restrict__ dx, float* __restrict__ g_part) {
    __shared__ float u_sh[2][CTL_TB];
    __shared__ float red[4][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int BL = B * L;
    const int blk = blockIdx.x;

    // direction norms
    float sp = 0.f, sr = 0.f;
    for (int j = tid; j <= D; j += blockDim.x) {
        sp = fmaf(w_phi[j], w_phi[j], sp);
        sr = fmaf(w_r[j], w_r[j], sr);
    }
    sp = wave_sum(sp);
    sr = wave_sum(sr);
    if (lane == 0) { red[0][wave] = sp; red[1][wave] = sr; }
    __syncthreads();
    float np = 0.f, nr = 0.f;
    for (int i = 0; i < nw; ++i) { np += red[0][i]; nr += red[1][i]; }
    const float inv_phi = 1.0f / sqrtf(np), inv_r = 1.0f / sqrtf(nr);
    const float sM = sqrtf((float)M);
    const float th_phi = tanhf(a_phi[0]), th_r = tanhf(a_r[0]);
    __syncthreads();

    // per-token u-bar (threads 0..CTL_TB-1, i.e. the first wave)
    if (tid < CTL_TB) {
        const int tok = blk * CTL_TB + tid;
        float uphi = 0.f, ur = 0.f, sdp = 0.f, scq = 0.f;
        if (tok < BL) {
            const int bb = tok / L, l = tok - bb * L;
            float cb = 0.f, dbr = 0.f;
            for (int t = 0; t < n_tiles; ++t) {
                const float2 v = reinterpret_cast<const float2*>(tok_part)[((size_t)bb * n_tiles + t) * L + l];
                cb += v.x;
                dbr += v.y;
            }
            const float p = p_sv[tok], r = r_sv[tok];
            const float r2 = r * r;
            const float q = r / (1.0f + r2);
            const float pbar = dbr * th_phi / sM;
            const float rbar = cb * th_r / sM * (1.0f - r2) / ((1.0f + r2) * (1.0f + r2));
            uphi = pbar * (1.0f - p * p);
            ur = rbar * (1.0f - r2);
            sdp = dbr * p;
            scq = cb * q;
        }
        u_sh[0][tid] = uphi;
        u_sh[1][tid] = ur;
        // bias column of x~ is 1: its gradient partial is sum u-bar
        const float s0 = wave_sum(uphi), s1 = wave_sum(ur), s2 = wave_sum(sdp), s3 = wave_sum(scq);
        if (tid == 0) {
            float* gp = g_part + (size_t)blk * (D + 2) * 2;
            gp[2 * D] = s0;
            gp[2 * D + 1] = s1;
            gp[2 * (D + 1)] = s2;
            gp[2 * (D + 1) + 1] = s3;
        }
    }
    __syncthreads();

    const int D8 = D >> 3;
    const int ntok = min(CTL_TB, BL - blk * CTL_TB);
    for (int j8 = tid; j8 < D8; j8 += blockDim.x) {  // 16-byte column group
        float wp[8], wr[8], gp[8], gr[8];
        {
            const float4* a = reinterpret_cast<const float4*>(w_phi) + 2 * j8;
            const float4* c = reinterpret_cast<const float4*>(w_r) + 2 * j8;
            const float4 a0 = a[0], a1 = a[1], c0 = c[0], c1 = c[1];
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wp[e] = av[e] * inv_phi;
                wr[e] = cv[e] * inv_r;
                gp[e] = 0.f;
                gr[e] = 0.f;
            }
        }
#pragma unroll 4
        for (int t = 0; t < ntok; ++t) {
            const size_t tok = (size_t)blk * CTL_TB + t;
            const float uphi = u_sh[0][t], ur = u_sh[1][t];
            const uint4 xv = x_sel[tok * D8 + j8];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            float xs[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { xs[2 * e] = bf16_lo(xw[e]); xs[2 * e + 1] = bf16_hi(xw[e]); }
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = fmaf(uphi, wp[e], ur * wr[e]);
                gp[e] = fmaf(uphi, xs[e], gp[e]);
                gr[e] = fmaf(ur, xs[e], gr[e]);
            }
            if (F32) {
                float4* q = reinterpret_cast<float4*>(dx) + (tok * D8 + j8) * 2;
                q[0] = make_float4(o[0], o[1], o[2], o[3]);
                q[1] = make_float4(o[4], o[5], o[6], o[7]);
            } else {
                reinterpret_cast<uint4*>(dx)[tok * D8 + j8] =
                    make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                               pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
            }
        }
        float4* out = reinterpret_cast<float4*>(g_part + ((size_t)blk * (D + 2) + 8 * j8) * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = make_float4(gp[2 * e], gr[2 * e], gp[2 * e + 1], gr[2 * e + 1]);
    }
}

// ----------------------------------------------------------------- K10 ---
// Level 1 of the parameter reductions, in FP64 and fixed order:
//   blocks [0, col_tiles): columns of g_part summed over a segment of token blocks
//   blocks [col_tiles, ...): modes of mode_part summed over a segment of chunks
constexpr int RED_THREADS = 256;

__global__ __launch_bounds__(RED_THREADS) void samu_param_reduce_kernel(
    int ncol, int n_blk, int seg_blk, int col_tiles, const float2* __restrict__ g_part,
    double2* __restrict__ g_seg, int M, int nchunks, int seg_chunk,
    const float2* __restrict__ mode_part, double2* __restrict__ mode_seg) {
    const int seg = blockIdx.y;
    // an empty segment (past the end) still writes zeros: level 2 sums all segments
    if ((int)blockIdx.x < col_tiles) {
        const int col = blockIdx.x * RED_THREADS + threadIdx.x;
        if (col >= ncol) return;
        const int b0 = min(n_blk, seg * seg_blk);
        const int b1 = min(n_blk, b0 + seg_blk);
        double sx = 0.0, sy = 0.0;
        for (int i = b0; i < b1; ++i) {
            const float2 v = g_part[(size_t)i * ncol + col];
            sx += v.x;
            sy += v.y;
        }
        g_seg[(size_t)seg * ncol + col] = make_double2(sx, sy);
    } else {
        const int m = (blockIdx.x - col_tiles) * RED_THREADS + threadIdx.x;
        if (m >= M) return;
        const int c0 = min(nchunks, seg * seg_chunk);
        const int c1 = min(nchunks, c0 + seg_chunk);
        double sx = 0.0, sy = 0.0;
        for (int i = c0; i < c1; ++i) {
            const float2 v = mode_part[(size_t)i * M + m];
            sx += v.x;
            sy += v.y;
        }
        mode_seg[(size_t)seg * M + m] = make_double2(sx, sy);
    }
}

// Level 2: block 0 finishes the direction and amplitude gradients (projection
// (g^ - w^ (w^ . g^)) / ||w||), the other blocks finish d nu, d theta.
constexpr int FIN_THREADS = 1024;

__global__ __launch_bounds__(FIN_THREADS) void samu_param_final_kernel(
    int D, int M, const float* __restrict__ w_phi, const float* __restrict__ w_r,
    const float* __restrict__ a_phi, const float* __restrict__ a_r,
    const double2* __restrict__ g_seg, int n_seg, const double2* __restrict__ mode_seg,
    int mode_nseg, float* __restrict__ dw_phi, float* __restrict__ dw_r,
    float* __restrict__ da_phi, float* __restrict__ da_r, float* __restrict__ dnu,
    float* __restrict__ dtheta) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (blockIdx.x > 0) {
        const int m = (blockIdx.x - 1) * FIN_THREADS + tid;
        if (m >= M) return;
        double sx = 0.0, sy = 0.0;
        for (int i = 0; i < mode_nseg; ++i) {
            const double2 v = mode_seg[(size_t)i * M + m];
            sx += v.x;
            sy += v.y;
        }
        dnu[m] = (float)sx;
        dtheta[m] = (float)sy;
        return;
    }
    extern __shared__ double gsh[];  // [D+2][2]
    __shared__ double red[4][FIN_THREADS / 64];
    const int ncol = D + 2;
    double nphi = 0.0, nr = 0.0, dphi = 0.0, dr = 0.0;
    for (int j = tid; j < ncol; j += FIN_THREADS) {
        double sx = 0.0, sy = 0.0;
        for (int i = 0; i < n_seg; ++i) {
            const double2 v = g_seg[(size_t)i * ncol + j];
            sx += v.x;
            sy += v.y;
        }
        gsh[2 * j] = sx;
        gsh[2 * j + 1] = sy;
        if (j <= D) {
            const double wp = w_phi[j], wr = w_r[j];
            nphi += wp * wp;
            nr += wr * wr;
            dphi += wp * sx;
            dr += wr * sy;
        }
    }
    nphi = wave_sum_d(nphi);
    nr = wave_sum_d(nr);
    dphi = wave_sum_d(dphi);
    dr = wave_sum_d(dr);
    if (lane == 0) { red[0][wave] = nphi; red[1][wave] = nr; red[2][wave] = dphi; red[3][wave] = dr; }
    __syncthreads();
    double Np = 0.0, Nr = 0.0, Dp = 0.0, Dr = 0.0;
    for (int i = 0; i < FIN_THREADS / 64; ++i) { Np += red[0][i]; Nr += red[1][i]; Dp += red[2][i]; Dr += red[3][i]; }
    const double np = sqrt(Np), nrr = sqrt(Nr);
    // w^ . g^ = (w . g^) / ||w||
    const double dotp = Dp / np, dotr = Dr / nrr;
    for (int j = tid; j <= D; j += FIN_THREADS) {
        const double whp = w_phi[j] / np, whr = w_r[j] / nrr;
        dw_phi[j] = (float)((gsh[2 * j] - whp * dotp) / np);
        dw_r[j] = (float)((gsh[2 * j + 1] - whr * dotr) / nrr);
    }
    if (tid == 0) {
        const double sM = sqrt((double)M);
        const double tp = tanh((double)a_phi[0]), tr = tanh((double)a_r[0]);
        da_phi[0] = (float)((1.0 - tp * tp) / sM * gsh[2 * (D + 1)]);
        da_r[0] = (float)((1.0 - tr * tr) / sM * gsh[2 * (D + 1) + 1]);
    }
}

}  // namespace

int samu_bwd_tiles(int M) { return (int)ceil_div(M, 64); }

hipError_t launch_samu_bwd_replay(const SamuParams& p, const Chunking& ch, const float* ctl,
                                  const float* entries, const float* carry_in, const void* dy,
                                  void* db, int db_f32, float* dz0, float* tok_part, int n_tiles,
                                  float* mode_part, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(p.M, BWD_THREADS), ch.C, ch.B);
#define BWD_CASE(KK, FF)                                                                             \
    LRS_LAUNCH(K_SAMU_BWD_REPLAY, (samu_bwd_replay_kernel<KK, FF>), grid, dim3(BWD_THREADS), 0, s, \
               p.L, p.M, ch.C, n_tiles, (const TokenCtl*)ctl, (const uint32_t*)p.b, p.nu, p.theta, \
               (const float2*)entries, (const float2*)carry_in, (const uint32_t*)dy, db,          \
               (float2*)dz0, tok_part, (float2*)mode_part)
    if (ch.K == 32) {
        if (db_f32) BWD_CASE(32, true); else BWD_CASE(32, false);
    } else {
        if (db_f32) BWD_CASE(16, true); else BWD_CASE(16, false);
    }
#undef BWD_CASE
    return hipGetLastError();
}

hipError_t launch_samu_ctl_bwd(const SamuParams& p, const float* p_sv, const float* r_sv,
                               const float* tok_part, int n_tiles, void* dx_sel, int dx_f32,
                               float* g_part, int tok_per_blk, hipStream_t s) {
    (void)tok_per_blk;
    const int BL = p.B * p.L;
    const int grid = (int)ceil_div(BL, CTL_TB);
    const int threads = (int)std::min<int64_t>(512, std::max<int64_t>(64, ceil_div(ceil_div(p.D, 8), 64) * 64));
    if (dx_f32)
        LRS_LAUNCH(K_SAMU_CTL_BWD, samu_ctl_bwd_kernel<true>, dim3(grid), dim3(threads), 0, s, p.B, p.L,
                   p.D, p.M, n_tiles, (const uint4*)p.x_sel, p.w_phi, p.w_r, p.a_phi, p.a_r, p_sv, r_sv,
                   tok_part, dx_sel, g_part);
    else
        LRS_LAUNCH(K_SAMU_CTL_BWD, samu_ctl_bwd_kernel<false>, dim3(grid), dim3(threads), 0, s, p.B, p.L,
                   p.D, p.M, n_tiles, (const uint4*)p.x_sel, p.w_phi, p.w_r, p.a_phi, p.a_r, p_sv, r_sv,
                   tok_part, dx_sel, g_part);
    return hipGetLastError();
}

int samu_ctl_tok_per_blk() { return CTL_TB; }

hipError_t launch_samu_param_reduce(const SamuParams& p, const Chunking& ch, const float* g_part,
                                    int n_blk, const float* mode_part, double* g_seg, int n_seg,
                                    double* mode_seg, hipStream_t s) {
    const int ncol = p.D + 2;
    const int seg_blk = (int)ceil_div(n_blk, n_seg);
    const int nchunks = ch.B * ch.C;
    const int seg_chunk = (int)ceil_div(nchunks, n_seg);
    const int col_tiles = (int)ceil_div(ncol, RED_THREADS);
    const int mode_tiles = (int)ceil_div(p.M, RED_THREADS);
    LRS_LAUNCH(K_SAMU_PARAM_REDUCE, samu_param_reduce_kernel, dim3(col_tiles + mode_tiles, n_seg),
               dim3(RED_THREADS), 0, s, ncol, n_blk, seg_blk, col_tiles, (const float2*)g_part,
               (double2*)g_seg, p.M, nchunks, seg_chunk, (const float2*)mode_part, (double2*)mode_seg);
    return hipGetLastError();
}

hipError_t launch_samu_param_final(const SamuParams& p, const Chunking& ch, const double* g_seg,
                                   int n_seg, const double* mode_seg, int mode_nseg, float* dw_phi,
                                   float* dw_r, float* da_phi, float* da_r, float* dnu,
                                   float* dtheta, hipStream_t s) {
    (void)ch;
    const size_t shmem = sizeof(double) * 2 * (size_t)(p.D + 2);
    const int grid = 1 + (int)ceil_div(p.M, FIN_THREADS);
    LRS_LAUNCH(K_SAMU_PARAM_FINAL, samu_param_final_kernel, dim3(grid), dim3(FIN_THREADS), shmem, s,
               p.D, p.M, p.w_phi, p.w_r, p.a_phi, p.a_r, (const double2*)g_seg, n_seg,
               (const double2*)mode_seg, mode_nseg, dw_phi, dw_r, da_phi, da_r, dnu, dtheta);
    return hipGetLastError();
}

}  // namespace lrs
