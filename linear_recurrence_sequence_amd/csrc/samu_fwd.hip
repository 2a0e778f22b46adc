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
// streams contiguous rows of the [B, L, M, 2] tensors.  The chunk's token
// controls (one 16-byte (E, C, S) record per token) are staged in LDS and
// read back as wave-uniform broadcasts.
#include "common.hpp"

namespace lrs {
namespace {

// ----------------------------------------------------------- controller ---
// One wave per CTL_TOK tokens: every lane loads 16 bytes (8 selector values)
// of each token row per 512-column slab, the wave reduces the two dot products
// and lanes 0..CTL_TOK-1 finish one token each.  The grid also writes the
// per-mode constant table (strided over all blocks).
#ifndef LRS_CTL_WAVES
#define LRS_CTL_WAVES 8
#endif
#ifndef LRS_CTL_TOK
#define LRS_CTL_TOK 8
#endif
constexpr int CTL_WAVES = LRS_CTL_WAVES;
constexpr int CTL_THREADS = 64 * CTL_WAVES;
constexpr int CTL_TOK = LRS_CTL_TOK;                // tokens per wave
constexpr int CTL_TOK_PER_BLOCK = CTL_WAVES * CTL_TOK;
#ifndef LRS_CTL_SLAB
#define LRS_CTL_SLAB 1
#endif
constexpr int CTL_SLAB = LRS_CTL_SLAB;  // 512-column slabs loaded together

__global__ __launch_bounds__(CTL_THREADS) void samu_controller_kernel(
    int L, int D, int M, int K, int K_last, int C, const uint4* __restrict__ x_sel, const float* __restrict__ w_phi,
    const float* __restrict__ w_r, const float* __restrict__ a_phi,
    const float* __restrict__ a_r, const float* __restrict__ nu, const float* __restrict__ theta,
    float* __restrict__ p_out, float* __restrict__ r_out, float2* __restrict__ u_out,
    TokenCtl* __restrict__ ctl, float4* __restrict__ mtab, float* __restrict__ inv_norm,
    float4* __restrict__ crec, uint4* __restrict__ clear, size_t n_clear) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const int D8 = D >> 3;  // 16-byte words per row
    // blocks are aligned to batch rows: block (b, jb) owns tokens
    // jb * CTL_TOK_PER_BLOCK ... of row b, so each chunk lies in one block
    const int nbr = (int)ceil_div(L, CTL_TOK_PER_BLOCK);
    const int b = blockIdx.x / nbr, jb = blockIdx.x - b * nbr;
    const int t0 = jb * CTL_TOK_PER_BLOCK + wave * CTL_TOK;  // token within the row
    const int tok0 = b * L + t0;                              // flat token
    float ap[CTL_TOK], ar[CTL_TOK];
#pragma unroll
    for (int q = 0; q < CTL_TOK; ++q) { ap[q] = 0.f; ar[q] = 0.f; }
    // squared direction norms from the weights the dot products load anyway
    // (every wave covers all D columns, so each wave forms the whole norm)
    float sp = 0.f, sr = 0.f;
    // CTL_SLAB column slabs of 512 selector columns per iteration, all their
    // loads issued before the arithmetic
    for (int j0 = lane; j0 < D8; j0 += 64 * CTL_SLAB) {
        uint4 xv[CTL_SLAB][CTL_TOK];
#pragma unroll
        for (int sl = 0; sl < CTL_SLAB; ++sl) {
            const int j = j0 + 64 * sl;
#pragma unroll
            for (int q = 0; q < CTL_TOK; ++q)
                xv[sl][q] = (j < D8 && t0 + q < L) ? x_sel[(size_t)(tok0 + q) * D8 + j]
                                                      : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int sl = 0; sl < CTL_SLAB; ++sl) {
            const int j = j0 + 64 * sl;
            if (j >= D8) break;
            const float4 wp0 = reinterpret_cast<const float4*>(w_phi)[2 * j];
            const float4 wp1 = reinterpret_cast<const float4*>(w_phi)[2 * j + 1];
            const float4 wr0 = reinterpret_cast<const float4*>(w_r)[2 * j];
            const float4 wr1 = reinterpret_cast<const float4*>(w_r)[2 * j + 1];
            const float wp[8] = {wp0.x, wp0.y, wp0.z, wp0.w, wp1.x, wp1.y, wp1.z, wp1.w};
            const float wr[8] = {wr0.x, wr0.y, wr0.z, wr0.w, wr1.x, wr1.y, wr1.z, wr1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sp = fmaf(wp[e], wp[e], sp);
                sr = fmaf(wr[e], wr[e], sr);
            }
#pragma unroll
            for (int q = 0; q < CTL_TOK; ++q) {
                const uint32_t xw[4] = {xv[sl][q].x, xv[sl][q].y, xv[sl][q].z, xv[sl][q].w};
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
    for (int q = 0; q < CTL_TOK; ++q) {
        const float sp_q = wave_sum(ap[q]), sr_q = wave_sum(ar[q]);
        if (lane == q) { up = sp_q; ur = sr_q; }
    }

    // The dot products above use the raw directions; the mode table comes
    // after the selector stream has been consumed rather than delaying its
    // first request.
    for (int m = blockIdx.x * CTL_THREADS + tid; m < M; m += gridDim.x * CTL_THREADS)
        store_mode(mtab, m, mode_const(nu[m], theta[m]), chunk_phase(theta[m], K), chunk_phase(theta[m], K_last));
    // direction norms over all D+1 entries: the wave's sum over columns
    // 0..D-1, then the bias entry
    const float np = fmaf(w_phi[D], w_phi[D], wave_sum(sp)), nr = fmaf(w_r[D], w_r[D], wave_sum(sr));
    const float inv_phi = 1.0f / sqrtf(np), inv_r = 1.0f / sqrtf(nr);
    if (inv_norm && blockIdx.x == 0) {
        // for the backward: 1/||w|| as used here (controller backward), and
        // the FP64 squared norms in a fixed order (parameter gradients)
        double sp2 = 0.0, sr2 = 0.0;
        for (int j = tid; j <= D; j += CTL_THREADS) {
            sp2 += (double)w_phi[j] * w_phi[j];
            sr2 += (double)w_r[j] * w_r[j];
        }
        sp2 = wave_sum_d(sp2);
        sr2 = wave_sum_d(sr2);
        __shared__ double dred[2][CTL_WAVES];
        if (lane == 0) {
            dred[0][wave] = sp2;
            dred[1][wave] = sr2;
        }
        __syncthreads();
        if (tid == 0) {
            double np2 = 0.0, nr2 = 0.0;
            for (int i = 0; i < CTL_WAVES; ++i) {
                np2 += dred[0][i];
                nr2 += dred[1][i];
            }
            inv_norm[0] = inv_phi;
            inv_norm[1] = inv_r;
            double* n2 = reinterpret_cast<double*>(inv_norm + 4);
            n2[0] = np2;
            n2[1] = nr2;
        }
    }
    const float amp_phi = tanhf(a_phi[0]) / sqrtf((float)M);
    const float amp_r = tanhf(a_r[0]) / sqrtf((float)M);
    const float bias_phi = w_phi[D], bias_r = w_r[D];

    const int tok = tok0 + lane;
    __shared__ float2 sed[CTL_TOK_PER_BLOCK];  // (E, d) of the block's tokens, for the chunk records
    if (lane < CTL_TOK && t0 + lane < L) {
        // x~ . w^ = (x_sel . w[0:D] + w[D]) / ||w||
        const float u_phi = (up + bias_phi) * inv_phi;
        const float u_r = (ur + bias_r) * inv_r;
        const float p = tanhf(u_phi);
        const float r = tanhf(u_r);
        const float q = r / (1.0f + r * r);
        const float d = amp_phi * p, c = amp_r * q;
        p_out[tok] = p;
        r_out[tok] = r;
        u_out[tok] = make_float2(u_phi, u_r);
        float sd, cd;
        sincosf(d, &sd, &cd);
        TokenCtl t;
        t.E = expf(c);
        t.C = cd;
        t.S = sd;
        t.d = d;
        ctl[tok] = t;
        sed[wave * CTL_TOK + lane] = make_float2(t.E, d);
    }
    if (crec) {  // uniform over the grid
        // the record of every chunk in this block: G_c = sum E_t and
        // D_c = sum d_t in token order, and (cos D_c, sin D_c)
        __syncthreads();
        const int nck = CTL_TOK_PER_BLOCK / K;
        const int tb = jb * CTL_TOK_PER_BLOCK + tid * K;  // the chunk's first token in the row
        if (tid < nck && tb < L) {
            const int kc = min(K, L - tb);
            float G = 0.f, Dd = 0.f;
            for (int i = 0; i < kc; ++i) {
                const float2 v = sed[tid * K + i];
                G += v.x;
                Dd += v.y;
            }
            float sD, cD;
            sincosf(Dd, &sD, &cD);
            crec[(size_t)b * C + tb / K] = make_float4(G, cD, sD, 0.f);
        }
    }
    // the single-pass forward's hand-off words start invalid (zero)
    for (size_t i = (size_t)blockIdx.x * CTL_THREADS + tid; i < n_clear; i += (size_t)gridDim.x * CTL_THREADS)
        clear[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ----------------------------------------- chunk and reverse summaries ---
template <int VM> struct Words;
// VM packed BF16 complex words of one lane; `row` is wave-uniform and `off`
// the lane's 32-bit word offset, so the load takes the scalar-base form.
template <> struct Words<1> {
    uint32_t w[1];
    __device__ void load(const uint32_t* row, int off) { w[0] = row[off]; }
};
template <> struct Words<2> {
    uint32_t w[2];
    __device__ void load(const uint32_t* row, int off) {
        uint2 v = *reinterpret_cast<const uint2*>(row + off);
        w[0] = v.x; w[1] = v.y;
    }
};
template <> struct Words<4> {
    uint32_t w[4];
    __device__ void load(const uint32_t* row, int off) {
        uint4 v = *reinterpret_cast<const uint4*>(row + off);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
};

#ifndef LRS_SUM_VM
#define LRS_SUM_VM 1
#endif
#ifndef LRS_REP_VM
#define LRS_REP_VM 1
#endif
constexpr int SUM_VM = LRS_SUM_VM;
constexpr int REP_VM = LRS_REP_VM;

// All drive words of one chunk for this lane, issued before anything else is
// scheduled: the recurrence is serial within a lane, so memory-level
// parallelism comes from requesting the whole chunk at once.  Only the last
// chunk of a sequence can be partial; full chunks take the branch-free path.
// REV: requested last token first, the order the reverse summary consumes
// them in (waits are in issue order).
template <int VM, int K, bool FULL, bool REV = false>
__device__ __forceinline__ void load_chunk(Words<VM> (&w)[K], const uint32_t* __restrict__ rows, int M,
                                           int off, int kc) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int i = REV ? K - 1 - j : j;
        if (FULL || i < kc) w[i].load(rows + (size_t)i * M, off);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One step of the forward summary (REV = false) or of the reverse conjugate
// summary (REV = true) for the VM modes of this lane: only the affine part B
// is carried; the chunk's transition product follows from (G_c, D_c).
template <int VM, bool REV>
__device__ __forceinline__ void summary_step(const ModeConst (&k)[VM], cf (&Bv)[VM], const TokenCtl& tc,
                                             const Words<VM>& dw) {
#pragma unroll
    for (int v = 0; v < VM; ++v) {
        const cf lam = mode_lambda(k[v], tc.E, tc.C, tc.S);
        const cf x = {bf16_lo(dw.w[v]), bf16_hi(dw.w[v])};
        if (!REV) Bv[v] = cfma(lam, Bv[v], x);                            // B -> lam B + x
        else Bv[v] = cmulc(lam, {Bv[v].re + x.re, Bv[v].im + x.im});     // B -> conj(lam) (x + B)
    }
}

// Chunk summary S_c (or, REV, the conjugate reverse summary of the chunk),
// one workgroup per (chunk, slice of modes), stored compressed: the affine
// part B per mode, and once per chunk (G_c, cos D_c, sin D_c) from which the
// prefix rebuilds the transition product of every mode (the closed form in
// common.hpp; the reverse product is its conjugate, so both directions write
// the same record).  The token controls of the chunk are requested first and
// staged in LDS; the drive loads follow as one batch.
template <int VM, int K, bool REV, bool FULL>
__device__ __forceinline__ void summary_chunk(TokenCtl (&sctl)[K], int L, int M, int C, int b, int c,
                                              int m0, bool active, const TokenCtl* __restrict__ ctl,
                                              const uint32_t* __restrict__ drive,
                                              const float4* __restrict__ mtab, float* __restrict__ summ,
                                              float4* __restrict__ chunk_rec) {
    const int s = c * K;
    const int kc = FULL ? K : L - s;
    const int mc = active ? m0 : M - VM;
    float4 tn = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((int)threadIdx.x < kc) tn = reinterpret_cast<const float4*>(ctl)[(size_t)b * L + s + threadIdx.x];
    // the mode constants first: the first step then waits for its own drive
    // word only, not for the whole chunk's
    ModeConst k[VM];
    cf Bv[VM];
#pragma unroll
    for (int v = 0; v < VM; ++v) {
        k[v] = load_mode(mtab, mc + v);
        Bv[v] = {0.f, 0.f};
    }
    Words<VM> w[K];
    load_chunk<VM, K, FULL, REV>(w, drive + ((size_t)b * L + s) * M, M, mc, kc);
    if ((int)threadIdx.x < kc) reinterpret_cast<float4*>(sctl)[threadIdx.x] = tn;
    __syncthreads();
    const int kq = opaque(kc);
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int i = REV ? K - 1 - j : j;
        if (i < kq) summary_step<VM, REV>(k, Bv, sctl[i], w[i]);
    }
    if (active) {
        float2* out = reinterpret_cast<float2*>(summ) + ((size_t)b * C + c) * M + m0;
#pragma unroll
        for (int v = 0; v < VM; ++v) out[v] = make_float2(Bv[v].re, Bv[v].im);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // G_c and D_c in token order, the same in both directions
        float G = 0.f, Dd = 0.f;
        for (int i = 0; i < kc; ++i) {
            G += sctl[i].E;
            Dd += sctl[i].d;
        }
        float sD, cD;
        sincosf(Dd, &sD, &cD);
        chunk_rec[(size_t)b * C + c] = make_float4(G, cD, sD, 0.f);
    }
}

// At least 4 waves per SIMD: otherwise the scheduler hoists every token's
// transition ahead of the serial chain and occupancy collapses.
template <int VM, int K, bool REV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void samu_summary_kernel(
    int L, int M, int C, const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
    const float4* __restrict__ mtab, float* __restrict__ summ, float4* __restrict__ chunk_rec) {
    __shared__ TokenCtl sctl[K];
    const int m0 = (blockIdx.x * blockDim.x + threadIdx.x) * VM;
    const int c = blockIdx.y, b = blockIdx.z;
    const bool active = m0 < M;
    if ((c + 1) * K <= L)
        summary_chunk<VM, K, REV, true>(sctl, L, M, C, b, c, m0, active, ctl, drive, mtab, summ, chunk_rec);
    else
        summary_chunk<VM, K, REV, false>(sctl, L, M, C, b, c, m0, active, ctl, drive, mtab, summ, chunk_rec);
}

// --------------------------------------------------------------- replay ---
// y row `row` (wave-uniform element index of the row start) at the lane's
// offset `off`, as VM complex values.
template <int VM, bool F32>
__device__ __forceinline__ void store_states(void* y, size_t row, int off, const cf (&z)[VM]) {
    if (F32) {
        float2* o = reinterpret_cast<float2*>(y) + row + off;
        if (VM == 4) {
            out_f32x4(o, z[0].re, z[0].im, z[1].re, z[1].im);
            out_f32x4(o + 2, z[2].re, z[2].im, z[3].re, z[3].im);
        } else if (VM == 2) {
            out_f32x4(o, z[0].re, z[0].im, z[1].re, z[1].im);
        } else {
#pragma unroll
            for (int v = 0; v < VM; ++v) out_f32x2(o + v, z[v].re, z[v].im);
        }
    } else {
        uint32_t* o = reinterpret_cast<uint32_t*>(y) + row + off;
        if (VM == 4) {
            out_u32x4(o, pack_bf16x2(z[0].re, z[0].im), pack_bf16x2(z[1].re, z[1].im),
                      pack_bf16x2(z[2].re, z[2].im), pack_bf16x2(z[3].re, z[3].im));
        } else if (VM == 2) {
            out_u32x2(o, pack_bf16x2(z[0].re, z[0].im), pack_bf16x2(z[1].re, z[1].im));
        } else {
#pragma unroll
            for (int v = 0; v < VM; ++v) out_u32(o + v, pack_bf16x2(z[v].re, z[v].im));
        }
    }
}

// Replay of one chunk from its entry state Q_c(init) = L_c(O_g(init)):
// y_t = z_t for every token; the last chunk also writes z_final.  The state
// entering each backward sub-chunk after the first goes to `mid`.
template <int VM, int K, bool F32, bool FULL>
__device__ __forceinline__ void replay_chunk(TokenCtl (&sctl)[K], int L, int M, int C, int b, int c,
                                             int m0, bool active, const TokenCtl* __restrict__ ctl,
                                             const uint32_t* __restrict__ drive,
                                             const float4* __restrict__ mtab,
                                             const float* __restrict__ entries, float* __restrict__ mid,
                                             void* __restrict__ y, float* __restrict__ z_final) {
    constexpr int NMID = samu_mid_states(K);
    const int s = c * K;
    const int kc = FULL ? K : L - s;
    const int mc = active ? m0 : M - VM;
    const size_t row0 = ((size_t)b * L + s) * M;  // wave-uniform
    float4 tn = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((int)threadIdx.x < kc) tn = reinterpret_cast<const float4*>(ctl)[(size_t)b * L + s + threadIdx.x];
    // the mode constants and the entry state first: the first token then
    // waits for its own drive word only, not for the whole chunk's
    ModeConst k[VM];
    cf z[VM];
    const float2* ent = reinterpret_cast<const float2*>(entries) + ((size_t)b * C + c) * M + mc;
#pragma unroll
    for (int v = 0; v < VM; ++v) {
        k[v] = load_mode(mtab, mc + v);
        const float2 e = ent[v];
        z[v] = {e.x, e.y};
    }
    Words<VM> w[K];
    load_chunk<VM, K, FULL>(w, drive + row0, M, mc, kc);
    if ((int)threadIdx.x < kc) reinterpret_cast<float4*>(sctl)[threadIdx.x] = tn;
    __syncthreads();
    const int kq = opaque(kc);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (i < kq) {
            const TokenCtl t = sctl[i];
#pragma unroll
            for (int v = 0; v < VM; ++v)
                z[v] = cfma(mode_lambda(k[v], t.E, t.C, t.S), z[v], {bf16_lo(w[i].w[v]), bf16_hi(w[i].w[v])});
            if (active) store_states<VM, F32>(y, row0 + (size_t)i * M, mc, z);
            if (NMID > 0 && (i + 1) % SAMU_BWD_SUB == 0 && i + 1 < K && active) {
                float2* md = reinterpret_cast<float2*>(mid) +
                             (((size_t)b * C + c) * NMID + (i + 1) / SAMU_BWD_SUB - 1) * M + mc;
#pragma unroll
                for (int v = 0; v < VM; ++v) md[v] = make_float2(z[v].re, z[v].im);
            }
        }
    }
    if (active && z_final && c == C - 1) {
        float2* zf = reinterpret_cast<float2*>(z_final) + (size_t)b * M + m0;
#pragma unroll
        for (int v = 0; v < VM; ++v) zf[v] = make_float2(z[v].re, z[v].im);
    }
}

template <int VM, int K, bool F32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void samu_replay_kernel(
    int L, int M, int C, const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
    const float4* __restrict__ mtab, const float* __restrict__ entries, float* __restrict__ mid,
    void* __restrict__ y, float* __restrict__ z_final) {
    __shared__ TokenCtl sctl[K];
    const int m0 = (blockIdx.x * blockDim.x + threadIdx.x) * VM;
    const int c = blockIdx.y, b = blockIdx.z;
    const bool active = m0 < M;
    // full chunks of workgroups whose lanes all hold modes take a copy with
    // the per-token lane masks folded away
    if ((c + 1) * K <= L && (int)((blockIdx.x + 1) * blockDim.x) * VM <= M)
        replay_chunk<VM, K, F32, true>(sctl, L, M, C, b, c, m0, true, ctl, drive, mtab, entries, mid, y,
                                       z_final);
    else if ((c + 1) * K <= L)
        replay_chunk<VM, K, F32, true>(sctl, L, M, C, b, c, m0, active, ctl, drive, mtab, entries, mid, y,
                                       z_final);
    else
        replay_chunk<VM, K, F32, false>(sctl, L, M, C, b, c, m0, active, ctl, drive, mtab, entries, mid, y,
                                        z_final);
}

// ------------------------------------------------ grouped (fused) path ---
// A workgroup owns one group of G consecutive chunks in processing order
// (forward: chunk q G + w; adjoint: chunk C - 1 - (q G + w)) and 64 modes:
// wave w handles chunk w of the group, lane l mode 64 blockIdx.x + l.  The
// group's chunk summaries meet in LDS, so the summary kernel composes U_g
// there, and the replays form L_c applied to the state entering the group
// there: neither the compose nor the expand pass of the three-kernel prefix
// runs, and the per-chunk entry states are never read back from memory.
// Every wave reaches the workgroup's single barrier, including those past
// the last chunk; all loads are issued unconditionally before it (a partial
// last chunk re-reads its last token row instead of branching).
constexpr int GRP_LANES = 64;

// (A, B) of this wave's chunk for this lane's mode, into the group's LDS
// table; A from the chunk record and the mode's chunk phasor.
__device__ __forceinline__ void group_put(float4* comp, int w, int lane, cf A, cf B) {
    comp[w * GRP_LANES + lane] = make_float4(A.re, A.im, B.re, B.im);
}

// The drive words of one chunk through its range-checked rows (tokens past a
// partial chunk's end read as 0 and are never used).
template <int K, bool REV>
__device__ __forceinline__ void load_chunk_clamped(Words<1> (&w)[K], const uint32_t* __restrict__ rows, int M,
                                                   int off, int kc) {
    const ChunkRows cr(rows, kc, M);
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int i = REV ? K - 1 - j : j;
        w[i].w[0] = cr.load(i, off);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The state entering each group comes from group_handoff (common.hpp): a
// fixed-order chain over segments of G groups, handed between workgroups
// through tagged words that the controller clears before every forward.
template <int K, bool F32, bool ALLACT>
__device__ __forceinline__ void gscan_body(float4* gdyn, int G, int L, int M, int C,
                                           const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
                                           const float4* __restrict__ mtab, const float4* __restrict__ chunk_rec,
                                           const float2* __restrict__ z0, uint64_t* __restrict__ pub,
                                           float2* __restrict__ entries, float* __restrict__ mid,
                                           void* __restrict__ y, float* __restrict__ z_final, int polls) {
    constexpr int NMID = samu_mid_states(K);
    float4* comp = gdyn;                   // [G][64] (A_c, B_c) of the group's chunks
    float4* look = gdyn + G * GRP_LANES;   // [G][64] what each wave read of the earlier groups
    TokenCtl* sctl = reinterpret_cast<TokenCtl*>(gdyn + 2 * G * GRP_LANES);
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int q = blockIdx.y, b = blockIdx.z, NG = gridDim.y;
    const int pc = q * G + w;
    const bool valid = pc < C;  // wave-uniform
    const int c = min(pc, C - 1);
    const int m = blockIdx.x * GRP_LANES + lane;
    const bool active = ALLACT || m < M;
    const int mc = active ? m : M - 1;
    const int s = c * K;
    const int kc = min(K, L - s);
    const size_t row0 = ((size_t)b * L + s) * M;  // wave-uniform
    sctl += w * K;

    // requests: the token controls, the mode constants, the chunk record,
    // then the chunk's drive words, held until the replay
    float4 tn = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < kc) tn = reinterpret_cast<const float4*>(ctl)[(size_t)b * L + s + lane];
    ModeConst k[1];
    k[0] = load_mode(mtab, mc);
    const float4 ph = mtab[MODE_REC * mc + (c == C - 1 ? 3 : 2)];
    const float4 rec = chunk_rec[(size_t)b * C + c];
    Words<1> wd[K];
    load_chunk_clamped<K, false>(wd, drive + row0, M, mc, kc);
    if (lane < kc) reinterpret_cast<float4*>(sctl)[lane] = tn;
    wave_lds_sync();
    const int kq = opaque(kc);
    // the controls through one vector-register base kept for the whole
    // chunk (an LDS read needs its address in a vector register)
    const TokenCtl* sv = sctl + opaque_v(0u);
    cf A = {1.f, 0.f}, Bv[1] = {{0.f, 0.f}};
    if (valid) {
#pragma unroll
        for (int i = 0; i < K; ++i)
            if (i < kq) summary_step<1, false>(k, Bv, sv[i], wd[i]);
        A = chunk_transition<false>(k[0].kappa, ph, rec);
    }
    group_put(comp, w, lane, A, Bv[0]);
    __syncthreads();

    const GroupChunks gc{chunk_rec + (size_t)b * C, mtab[MODE_REC * mc + 2], mtab[MODE_REC * mc + 3], k[0].kappa, C};
    const float4 gin = group_handoff<false>(comp, look, G, w, lane, q, NG, M, mc, active,
                                            z0 ? z0 + (size_t)b * M : nullptr,
                                            pub + (size_t)b * NG * SCAN_PUB_WORDS * M, gc, polls);
    if (!valid) return;
    // the mode constants again (a fresh load, not registers held across the
    // hand-off)
    const ModeConst k2 = load_mode(mtab, (int)opaque_v((uint32_t)mc));
    // the state entering this chunk: L_c applied to the state entering the group
    cf z = {gin.x, gin.y};
    for (int j = 0; j < w; ++j) {
        const float4 f = comp[j * GRP_LANES + lane];
        z = cfma({f.x, f.y}, z, {f.z, f.w});
    }
    if (active) entries[((size_t)b * C + c) * M + m] = make_float2(z.re, z.im);
    const ChunkOut yo(reinterpret_cast<char*>(y) + row0 * (F32 ? 8 : 4), kc, M, F32 ? 8 : 4);
    const uint32_t yoff = (uint32_t)mc * (F32 ? 8u : 4u);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (i < kq) {
            const TokenCtl t = sv[i];
            // the word again, not the summary's unpacked pair kept live since
            const uint32_t xw = opaque_v(wd[i].w[0]);
            z = cfma(mode_lambda(k2, t.E, t.C, t.S), z, {bf16_lo(xw), bf16_hi(xw)});
            if (active) {
                if (F32) yo.f32x2(i, yoff, z.re, z.im);
                else yo.u32(i, yoff, pack_bf16x2(z.re, z.im));
            }
            if (NMID > 0 && (i + 1) % SAMU_BWD_SUB == 0 && i + 1 < K && active)
                reinterpret_cast<float2*>(mid)[(((size_t)b * C + c) * NMID + (i + 1) / SAMU_BWD_SUB - 1) * M + mc] =
                    make_float2(z.re, z.im);
        }
    }
    if (active && z_final && c == C - 1)
        reinterpret_cast<float2*>(z_final)[(size_t)b * M + m] = make_float2(z.re, z.im);
}

template <int K, bool F32>
__global__ __launch_bounds__(GRP_LANES * SAMU_GROUP_MAX) __attribute__((amdgpu_waves_per_eu(4, 8))) void
samu_gscan_kernel(int L, int M, int C, int G, const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
                  const float4* __restrict__ mtab, const float4* __restrict__ chunk_rec,
                  const float2* __restrict__ z0, uint64_t* __restrict__ pub, float2* __restrict__ entries,
                  float* __restrict__ mid, void* __restrict__ y, float* __restrict__ z_final, int polls) {
    extern __shared__ float4 gdyn[];
    if ((int)(blockIdx.x + 1) * GRP_LANES <= M)  // uniform over the workgroup
        gscan_body<K, F32, true>(gdyn, G, L, M, C, ctl, drive, mtab, chunk_rec, z0, pub, entries, mid, y, z_final,
                                 polls);
    else
        gscan_body<K, F32, false>(gdyn, G, L, M, C, ctl, drive, mtab, chunk_rec, z0, pub, entries, mid, y, z_final,
                                  polls);
}

inline int mode_block(int M, int VM) {
    const int lanes = (int)ceil_div(M, VM);
    return lanes >= 256 ? 256 : (int)ceil_div(lanes, 64) * 64;
}

}  // namespace

hipError_t launch_samu_controller(const SamuParams& p, const Chunking& ch, float* p_out, float* r_out,
                                  float* u_out, float* ctl, float* mtab, float* inv_norm, float* crec,
                                  void* clear, size_t clear_bytes, hipStream_t s) {
    static_assert(CTL_TOK_PER_BLOCK % 32 == 0, "chunks of 16 and 32 tokens must lie in one block");
    const int grid = p.B * (int)ceil_div(p.L, CTL_TOK_PER_BLOCK);
    const int K_last = p.L - (ch.C - 1) * ch.K;
    LRS_LAUNCH(K_SAMU_CONTROLLER, samu_controller_kernel, dim3(grid), dim3(CTL_THREADS), 0, s,
               p.L, p.D, p.M, ch.K, K_last, ch.C, (const uint4*)p.x_sel, p.w_phi, p.w_r, p.a_phi, p.a_r, p.nu,
               p.theta, p_out, r_out, (float2*)u_out, (TokenCtl*)ctl, (float4*)mtab, inv_norm, (float4*)crec,
               (uint4*)clear, clear ? clear_bytes / 16 : (size_t)0);
    return hipGetLastError();
}

hipError_t launch_samu_summary(const SamuParams& p, const Chunking& ch, const float* ctl,
                               const float* mtab, const void* drive, bool reverse, float* summ,
                               float* chunk_rec, hipStream_t s) {
    const int blk = mode_block(p.M, SUM_VM);
    const dim3 grid((unsigned)ceil_div(ceil_div(p.M, SUM_VM), blk), ch.C, ch.B);
    const int id = reverse ? K_SAMU_REV_SUMMARY : K_SAMU_SUMMARY;
#define SUMMARY_CASE(KK, RR)                                                                        \
    LRS_LAUNCH(id, (samu_summary_kernel<SUM_VM, KK, RR>), grid, dim3(blk), 0, s, p.L, p.M, ch.C, \
               (const TokenCtl*)ctl, (const uint32_t*)drive, (const float4*)mtab, summ,           \
               (float4*)chunk_rec)
    if (ch.K == 32) {
        if (reverse) SUMMARY_CASE(32, true); else SUMMARY_CASE(32, false);
    } else {
        if (reverse) SUMMARY_CASE(16, true); else SUMMARY_CASE(16, false);
    }
#undef SUMMARY_CASE
    return hipGetLastError();
}

hipError_t launch_samu_replay(const SamuParams& p, const Chunking& ch, const float* ctl,
                              const float* mtab, const float* entries, float* mid, void* y, int y_f32,
                              float* z_final, hipStream_t s) {
    const int blk = mode_block(p.M, REP_VM);
    const dim3 grid((unsigned)ceil_div(ceil_div(p.M, REP_VM), blk), ch.C, ch.B);
#define REPLAY_CASE(KK, FF)                                                                       \
    LRS_LAUNCH(K_SAMU_REPLAY, (samu_replay_kernel<REP_VM, KK, FF>), grid, dim3(blk), 0, s, p.L, \
               p.M, ch.C, (const TokenCtl*)ctl, (const uint32_t*)p.b, (const float4*)mtab,       \
               entries, mid, y, z_final)
    if (ch.K == 32) {
        if (y_f32) REPLAY_CASE(32, true); else REPLAY_CASE(32, false);
    } else {
        if (y_f32) REPLAY_CASE(16, true); else REPLAY_CASE(16, false);
    }
#undef REPLAY_CASE
    return hipGetLastError();
}

static size_t samu_group_lds_bytes(int G, int K) { return (size_t)G * GRP_LANES * sizeof(float4) + (size_t)G * K * sizeof(TokenCtl); }



}  // namespace lrs

namespace lrs {
size_t samu_gscan_pub_bytes(const Chunking& ch, int M) {
    return (size_t)ch.B * ch.NG * SCAN_PUB_WORDS * M * sizeof(uint64_t);
}

hipError_t launch_samu_gscan(const SamuParams& p, const Chunking& ch, const float* ctl, const float* mtab,
                             const float* chunk_rec, void* pub, float* entries, float* mid, void* y, int y_f32,
                             float* z_final, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(p.M, GRP_LANES), ch.NG, ch.B);
    const dim3 block(GRP_LANES * ch.G);
    const size_t lds = (size_t)2 * ch.G * GRP_LANES * sizeof(float4) + (size_t)ch.G * ch.K * sizeof(TokenCtl);
#define GSCAN_CASE(KK, FF)                                                                                     \
    LRS_LAUNCH(K_SAMU_FWD_SCAN, (samu_gscan_kernel<KK, FF>), grid, block, lds, s, p.L, p.M, ch.C, ch.G,       \
               (const TokenCtl*)ctl, (const uint32_t*)p.b, (const float4*)mtab, (const float4*)chunk_rec,      \
               (const float2*)p.z0, (uint64_t*)pub, (float2*)entries, mid, y, z_final, handoff_poll_limit())
    if (ch.K == 32) {
        if (y_f32) GSCAN_CASE(32, true); else GSCAN_CASE(32, false);
    } else {
        if (y_f32) GSCAN_CASE(16, true); else GSCAN_CASE(16, false);
    }
#undef GSCAN_CASE
    return hipGetLastError();
}
}  // namespace lrs
