// samu_decode.hip -- one SAMU generation step for a batch of sequences, in a
// single launch.
//
// Page 'Griffin 第 4、5 节 H800 对照协议', 'SAMU 的固定方程': the decode kernel
// performs the control projection, the transition rebuild, the FP32 state
// update and the BF16 output in one launch.  The equations are those of page
// 'SAMU 与 RG-LRU 的 H800 训练性能对比', section 05, for one token:
//   u = x~ . w^ (x~ = [x_sel; 1], w^ = w/||w|| over all D+1 entries),
//   p = tanh(u_phi), r = tanh(u_r), q = r/(1+r^2),
//   d = tanh(a_phi)/sqrt(M) p, c = tanh(a_r)/sqrt(M) q,
//   lambda_m = exp(-nu_m e^c) [(cos th_m cos d - sin th_m sin d) + i (...)],
//   z' = lambda z + b,  y = z'.
//
// Grid (ceil(M / NT), B) with NT = 256 threads (512 from 128 rows up): each
// workgroup forms the two dot products (and, without a prepared table, the
// two direction norms) of its batch row, 16 bytes of the row per thread and
// step, then NT lanes advance one mode each.  Every mode block repeats the
// row's small reduction, which measured faster than one workgroup per row
// (1024 threads), and faster than several rows per workgroup sharing the
// direction loads (the rows then run one after another in each workgroup).
// Sums run in a fixed order for a given batch size and width, so a step is
// bitwise reproducible.
#include "common.hpp"

namespace lrs {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;

// TAB: the mode constants, 1/||w|| and tanh(a)/sqrt(M) come from a table
// written once by samu_decode_prepare_kernel (no FP64 phasor, no norm
// reduction and no amplitude tanh per step).
template <bool F32, bool TAB, int NT>
__global__ __launch_bounds__(NT) void samu_decode_kernel(
    int B, int D, int M, const uint32_t* __restrict__ x_sel, const uint32_t* __restrict__ drive,
    const float* __restrict__ w_phi, const float* __restrict__ w_r, const float* __restrict__ a_phi,
    const float* __restrict__ a_r, const float* __restrict__ nu, const float* __restrict__ theta,
    const float4* __restrict__ table, const float2* z_in, float2* z_out, void* __restrict__ y) {
    constexpr int R = 1;  // batch rows per workgroup
    constexpr int NW = NT / 64;
    __shared__ float red[2 * R + 2][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b0 = blockIdx.y * R;
    const int W = D / 2;  // selector words per row

    // this lane's mode in each row: its inputs are requested first and its
    // constant phasor is formed (or loaded) while the reduction is in flight
    const int m = blockIdx.x * NT + tid;
    const bool act = m < M;
    const int mc = act ? m : M - 1;
    float2 zr[R];
    uint32_t bw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const size_t i = (size_t)min(b0 + r, B - 1) * M + mc;
        zr[r] = z_in ? z_in[i] : make_float2(0.f, 0.f);
        bw[r] = drive[i];
    }
    ModeConst k;
    float4 inv = make_float4(0.f, 0.f, 0.f, 0.f);
    float nu_m = 0.f, th_m = 0.f;
    if (TAB) {
        k = load_mode(table, mc);
        inv = table[(size_t)M * MODE_REC];
    } else {
        nu_m = nu[mc];
        th_m = theta[mc];
    }

    // dot products over 8 selector values (16 bytes) per thread and step;
    // each direction chunk is loaded once for the R rows
    float sp[R], sr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { sp[r] = 0.f; sr[r] = 0.f; }
    float np = 0.f, nr = 0.f;
    const int W4 = W >> 2;  // 16-byte selector pieces per row (D % 8 == 0)
    for (int j = tid; j < W4; j += NT) {
        uint4 xv[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            xv[r] = reinterpret_cast<const uint4*>(x_sel + (size_t)min(b0 + r, B - 1) * W)[j];
        const float4 p0 = reinterpret_cast<const float4*>(w_phi)[2 * j];
        const float4 p1 = reinterpret_cast<const float4*>(w_phi)[2 * j + 1];
        const float4 q0 = reinterpret_cast<const float4*>(w_r)[2 * j];
        const float4 q1 = reinterpret_cast<const float4*>(w_r)[2 * j + 1];
        const float wp[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        const float wr[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t xw[4] = {xv[r].x, xv[r].y, xv[r].z, xv[r].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sp[r] = fmaf(bf16_lo(xw[e]), wp[2 * e], sp[r]);
                sp[r] = fmaf(bf16_hi(xw[e]), wp[2 * e + 1], sp[r]);
                sr[r] = fmaf(bf16_lo(xw[e]), wr[2 * e], sr[r]);
                sr[r] = fmaf(bf16_hi(xw[e]), wr[2 * e + 1], sr[r]);
            }
        }
        if (!TAB) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                np = fmaf(wp[e], wp[e], np);
                nr = fmaf(wr[e], wr[e], nr);
            }
        }
    }
    if (tid == 0) {  // the constant 1 of x~ and the bias slot of each direction
        const float bp = w_phi[D], br = w_r[D];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            sp[r] += bp;
            sr[r] += br;
        }
        np = fmaf(bp, bp, np);
        nr = fmaf(br, br, nr);
    }
    if (!TAB) k = mode_const(nu_m, th_m);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        sp[r] = wave_sum(sp[r]);
        sr[r] = wave_sum(sr[r]);
    }
    if (!TAB) {
        np = wave_sum(np);
        nr = wave_sum(nr);
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            red[2 * r][wave] = sp[r];
            red[2 * r + 1][wave] = sr[r];
        }
        red[2 * R][wave] = np;
        red[2 * R + 1][wave] = nr;
    }
    __syncthreads();
    float Np = 0.f, Nr = 0.f;
    if (!TAB) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            Np += red[2 * R][w];
            Nr += red[2 * R + 1][w];
        }
    }
    const float sM = sqrtf((float)M);
    const float amp_p = TAB ? inv.z : tanhf(a_phi[0]) / sM;
    const float amp_r = TAB ? inv.w : tanhf(a_r[0]) / sM;
    if (!act) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (b0 + r >= B) break;  // uniform over the workgroup
        float Sp = 0.f, Sr = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            Sp += red[2 * r][w];
            Sr += red[2 * r + 1][w];
        }
        const float p = tanhf(TAB ? Sp * inv.x : Sp / sqrtf(Np));
        const float rr = tanhf(TAB ? Sr * inv.y : Sr / sqrtf(Nr));
        const float q = rr / (1.0f + rr * rr);
        const float d = amp_p * p;
        const float c = amp_r * q;
        const float E = expf(c);
        float S, Cd;
        sincosf(d, &S, &Cd);
        const cf lam = mode_lambda(k, E, Cd, S);
        const cf z = cfma(lam, {zr[r].x, zr[r].y}, {bf16_lo(bw[r]), bf16_hi(bw[r])});
        const size_t i = (size_t)(b0 + r) * M + mc;
        z_out[i] = make_float2(z.re, z.im);
        if (F32) reinterpret_cast<float2*>(y)[i] = make_float2(z.re, z.im);
        else reinterpret_cast<uint32_t*>(y)[i] = pack_bf16x2(z.re, z.im);
    }
}

// The table of samu_decode_kernel<.., true>: the per-mode constant records
// (the layout of the scan's mode table; its chunk phasors are not used here)
// and (1/||w_phi||, 1/||w_r||, tanh(a_phi)/sqrt(M), tanh(a_r)/sqrt(M)), the
// norms over all D+1 entries summed in a fixed order.
__global__ __launch_bounds__(DEC_THREADS) void samu_decode_prepare_kernel(int D, int M, const float* __restrict__ w_phi,
                                                                          const float* __restrict__ w_r,
                                                                          const float* __restrict__ a_phi,
                                                                          const float* __restrict__ a_r,
                                                                          const float* __restrict__ nu,
                                                                          const float* __restrict__ theta,
                                                                          float4* __restrict__ table) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = blockIdx.x * DEC_THREADS + tid;
    if (m < M) {
        const ChunkPhase one = chunk_phase(theta[m], 1);
        store_mode(table, m, mode_const(nu[m], theta[m]), one, one);
    }
    if (blockIdx.x != 0) return;
    __shared__ float red[2][DEC_WAVES];
    float np = 0.f, nr = 0.f;
    for (int j = tid; j <= D; j += DEC_THREADS) {
        np = fmaf(w_phi[j], w_phi[j], np);
        nr = fmaf(w_r[j], w_r[j], nr);
    }
    np = wave_sum(np);
    nr = wave_sum(nr);
    if (lane == 0) {
        red[0][wave] = np;
        red[1][wave] = nr;
    }
    __syncthreads();
    if (tid == 0) {
        float Np = 0.f, Nr = 0.f;
        for (int w = 0; w < DEC_WAVES; ++w) {
            Np += red[0][w];
            Nr += red[1][w];
        }
        const float sM = sqrtf((float)M);
        table[(size_t)M * MODE_REC] =
            make_float4(1.0f / sqrtf(Np), 1.0f / sqrtf(Nr), tanhf(a_phi[0]) / sM, tanhf(a_r[0]) / sM);
    }
}

}  // namespace

size_t samu_decode_table_floats(int M) { return ((size_t)M * MODE_REC + 1) * 4; }

hipError_t launch_samu_decode_prepare(int D, const float* w_phi, const float* w_r, const float* a_phi,
                                      const float* a_r, const float* nu, const float* theta, float* table,
                                      hipStream_t s) {
    const int M = D / 2;
    LRS_LAUNCH(K_SAMU_DECODE, samu_decode_prepare_kernel, dim3((unsigned)ceil_div(M, DEC_THREADS)),
               dim3(DEC_THREADS), 0, s, D, M, w_phi, w_r, a_phi, a_r, nu, theta, (float4*)table);
    return hipGetLastError();
}

hipError_t launch_samu_decode(int B, int D, const void* x_sel, const void* b, const float* w_phi,
                              const float* w_r, const float* a_phi, const float* a_r, const float* nu,
                              const float* theta, const float* table, const float* z_in, float* z_out, void* y,
                              int y_f32, hipStream_t s) {
    const int M = D / 2;
    // 512-thread workgroups from 128 rows up (half as many workgroups, each
    // row's reduction shared by 512 modes): measured faster at B = 256 (4.0
    // against 4.4 us per step from a graph), slower below 128 rows
    const int NT = B >= 128 ? 512 : DEC_THREADS;
    const dim3 grid((unsigned)ceil_div(M, NT), (unsigned)B);
#define DEC_CASE(FF, TT, N)                                                                                 \
    LRS_LAUNCH(K_SAMU_DECODE, (samu_decode_kernel<FF, TT, N>), grid, dim3(N), 0, s, B, D, M,               \
               (const uint32_t*)x_sel, (const uint32_t*)b, w_phi, w_r, a_phi, a_r, nu, theta,              \
               (const float4*)table, (const float2*)z_in, (float2*)z_out, y)
#define DEC_SIZES(FF, TT) \
    if (NT == 512) DEC_CASE(FF, TT, 512); else DEC_CASE(FF, TT, DEC_THREADS);
    if (table) {
        if (y_f32) { DEC_SIZES(true, true) } else { DEC_SIZES(false, true) }
    } else {
        if (y_f32) { DEC_SIZES(true, false) } else { DEC_SIZES(false, false) }
    }
#undef DEC_SIZES
#undef DEC_CASE
    return hipGetLastError();
}

}  // namespace lrs
