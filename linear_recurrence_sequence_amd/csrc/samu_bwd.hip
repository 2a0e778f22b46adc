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
// No atomic accumulation: every sum has a fixed order (the single-pass scan
// hands whole words between workgroups in an order fixed by the group
// index), so results are bitwise reproducible run to run.
#include "common.hpp"

namespace lrs {
namespace {

// ------------------------------------------------------ backward replay ---
// One lane per mode, one workgroup per (chunk, 256 modes).  The chunk is
// handled as K/H sub-chunks of H tokens, last one first, each from the state
// entering it (the chunk's saved entry state, or the saved mid state the
// forward replay kept): a sub-chunk recomputes lambda_t and
// w_t = lambda_t z_{t-1} for its H tokens and runs the adjoint over them in
// reverse, starting from the cotangent carried in from the following chunk.
// All drive words and the last sub-chunk's cotangent words are requested
// before any math, right after the saved states, in the order the sub-chunks
// consume them; each earlier sub-chunk requests its cotangent words as it
// starts.  The per-token partial sums of a wave are
// reduced through a padded LDS transpose (conflict-free both ways), one
// sub-chunk at a time.
constexpr int BWD_THREADS = 256;
#ifndef LRS_BWD_WAVES
#define LRS_BWD_WAVES 3  // waves per SIMD the register budget is sized for
#endif

// Requests of one chunk of the backward replay, in the order it consumes
// them: the states entering each sub-chunk (the chunk's saved entry state and
// the mid states the forward replay kept; those of sub-chunks past a partial
// chunk's end are never used), the last sub-chunk's drive words forward in
// time, then its cotangent words backward.  The cotangent words of the earlier
// sub-chunks are requested when their sub-chunk starts: holding them through
// the last sub-chunk would take the kernel past 128 VGPRs, i.e. from 4 to 3
// waves per SIMD, which costs more than the latency the early request hides.
// Past a partial chunk's end (token i >= kc) a load is skipped (CLAMP false:
// the word reads as zero) or re-reads token kc - 1 (CLAMP true: no branch;
// the word is never used).  The CLAMP form serves the single-pass backward,
// which reads each word once, so its loads carry the non-temporal hint.
template <int K, int H, bool FULL, bool CLAMP, bool GW = true>
__device__ __forceinline__ void bwd_issue(cf (&ck)[K / H], uint32_t (&bw)[K], uint32_t (&gw)[K], int kc,
                                          size_t row0, int M, int mm, size_t bc,
                                          const float2* __restrict__ entries, const float2* __restrict__ mid,
                                          const uint32_t* __restrict__ drive, const uint32_t* __restrict__ dy) {
    constexpr int NH = K / H;
    {
        const float2 e0 = entries[bc * M + mm];
        ck[0] = {e0.x, e0.y};
#pragma unroll
        for (int h = 1; h < NH; ++h) {
            const float2 v = mid[(bc * (NH - 1) + h - 1) * M + mm];
            ck[h] = {v.x, v.y};
        }
    }
#pragma unroll
    for (int h = NH - 1; h >= 0; --h) {
#pragma unroll
        for (int j = 0; j < H; ++j) {
            const int i = h * H + j;
            if (CLAMP) bw[i] = __builtin_nontemporal_load(&(drive + row0 + (size_t)min(i, kc - 1) * M)[mm]);
            else if (FULL) bw[i] = (drive + row0 + (size_t)i * M)[mm];
            else bw[i] = i < kc ? (drive + row0 + (size_t)i * M)[mm] : 0u;
        }
        if (!GW || h != NH - 1) continue;  // earlier sub-chunks: requested when they start
#pragma unroll
        for (int j = H - 1; j >= 0; --j) {
            const int i = h * H + j;
            if (CLAMP) gw[i] = __builtin_nontemporal_load(&(dy + row0 + (size_t)min(i, kc - 1) * M)[mm]);
            else if (FULL) gw[i] = (dy + row0 + (size_t)i * M)[mm];
            else gw[i] = i < kc ? (dy + row0 + (size_t)i * M)[mm] : 0u;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// The adjoint over one chunk, sub-chunk by sub-chunk, last one first, from
// the cotangent `carry` arriving after the chunk's last token; `sctl` holds
// the chunk's token controls.  FULL = the chunk has all K tokens (only the
// last chunk of a sequence may not), which keeps the common path free of
// per-token branches.  The per-token partial sums of a wave are reduced
// through its own padded LDS rows `lds_w` (conflict-free both ways); WSYNC
// orders that traffic with wave-local fences (every wave of the workgroup
// on its own chunk) instead of workgroup barriers.  CLAMP: one copy of the
// code for full and partial chunks alike -- loads past a partial chunk's end
// re-read its last token and every use is guarded by the token count.
// STASH: the first sub-chunk's state is read from ck0_lds, so ck[0] need not
// stay in a register through the later sub-chunks.  RH: tokens per partial-
// sum transpose (the rows hold RH tokens).  DYS: the cotangent words of the
// earlier sub-chunks come from the lane's LDS slots dy_lds[i * 64] (written
// by the caller) instead of a second read from memory.  BST: db goes out
// through a buffer descriptor over the chunk's rows (ChunkOut).
template <int K, int H, bool F32, bool FULL, bool WSYNC, bool CLAMP = false, bool STASH = false, int RH = H,
          bool DYS = false, bool BST = false>
__device__ __forceinline__ void bwd_body(float* lds_w, const TokenCtl* sctl, const ModeConst& k, bool active,
                                         int lane, int tile, int n_tiles, int L, int M, int b, int s, int kc,
                                         size_t row0, int mm, const uint32_t* __restrict__ dy, void* __restrict__ db,
                                         float* __restrict__ tok_part, const cf (&ck)[K / H], const uint32_t (&bw)[K],
                                         uint32_t (&gw)[K], cf& carry, float& acc_nu, float& acc_th,
                                         const float2* ck0_lds = nullptr, const uint32_t* dy_lds = nullptr) {
    constexpr int NH = K / H;
    static_assert(NH == 1 || (H == SAMU_BWD_SUB && NH - 1 == samu_mid_states(K)),
                  "sub-chunks must match the forward's mid states");
    static_assert(H % RH == 0 && 64 % (2 * RH) == 0, "transpose blocks");
    constexpr int NV = 2 * RH;
    constexpr int PAD = NV + 1;
    const int kq = opaque(kc);
    float* row = &lds_w[lane * PAD];
    const ChunkOut dbo(reinterpret_cast<char*>(db) + row0 * (F32 ? 8 : 4), kc, M, F32 ? 8 : 4);
    const uint32_t dboff = (uint32_t)mm * (F32 ? 8u : 4u);
#pragma unroll
    for (int h = NH - 1; h >= 0; --h) {
        const int i0 = h * H;
        if (!FULL && i0 >= kc) continue;  // uniform over the wave (and, unless WSYNC, the workgroup)
        if (h != NH - 1) {
#pragma unroll
            for (int j = H - 1; j >= 0; --j) {
                const int i = i0 + j;
                if (DYS) gw[i] = dy_lds[i * 64];
                else if (CLAMP) gw[i] = (dy + row0 + (size_t)min(i, kc - 1) * M)[mm];
                else gw[i] = (FULL || i < kc) ? (dy + row0 + (size_t)i * M)[mm] : 0u;
            }
        }
        cf lam[H], wz[H];
        {
            cf z = ck[h];
            if (STASH && h == 0) {  // the entry state, kept in LDS meanwhile
                const float2 e0 = *ck0_lds;
                z = {e0.x, e0.y};
            }
#pragma unroll
            for (int j = 0; j < H; ++j) {
                if (i0 + j < kq) {
                    const TokenCtl t = sctl[i0 + j];
                    lam[j] = mode_lambda(k, t.E, t.C, t.S);
                    wz[j] = cmul(lam[j], z);
                    z = {wz[j].re + bf16_lo(bw[i0 + j]), wz[j].im + bf16_hi(bw[i0 + j])};
                }
            }
        }
#pragma unroll
        for (int j = H - 1; j >= 0; --j) {
            float pr = 0.f, pi = 0.f;
            if (i0 + j < kq) {
                const size_t rowj = row0 + (size_t)(i0 + j) * M;
                const float E = sctl[i0 + j].E;
                const cf gg = {bf16_lo(gw[i0 + j]) + carry.re, bf16_hi(gw[i0 + j]) + carry.im};
                if (active) {
                    if (BST) {
                        if (F32) dbo.f32x2(i0 + j, dboff, gg.re, gg.im);
                        else dbo.u32(i0 + j, dboff, pack_bf16x2(gg.re, gg.im));
                    } else if (F32) {
                        out_f32x2(reinterpret_cast<float2*>(db) + rowj + mm, gg.re, gg.im);
                    } else {
                        out_u32(reinterpret_cast<uint32_t*>(db) + rowj + mm, pack_bf16x2(gg.re, gg.im));
                    }
                }
                // gamma = g conj(w)
                const float gre = fmaf(gg.re, wz[j].re, gg.im * wz[j].im);
                const float gim = fmaf(gg.im, wz[j].re, -gg.re * wz[j].im);
                acc_nu = fmaf(E, gre, acc_nu);
                acc_th += gim;
                pr = k.nu * gre;
                pi = gim;
                carry = cmulc(lam[j], gg);
            }
            if (!active) { pr = 0.f; pi = 0.f; }
            row[2 * (j % RH)] = pr;
            row[2 * (j % RH) + 1] = pi;
            if (j % RH != 0) continue;
            if (WSYNC) wave_lds_sync(); else __syncthreads();
            // column col (token j + col/2, component col%2) summed over the
            // wave's 64 modes: 64/NV lanes per column, NV rows each, then a
            // butterfly
            {
                const int col = lane % NV, grp = lane / NV;
                const float* src = &lds_w[grp * NV * PAD + col];
                float acc = 0.f;
#pragma unroll
                for (int r = 0; r < NV; ++r) acc += src[r * PAD];
#pragma unroll
                for (int o = NV; o < 64; o <<= 1) acc += __shfl_xor(acc, o);
                const int t = i0 + j + (col >> 1);
                if (grp == 0 && t < kc && tile < n_tiles) {
                    if ((col & 1) == 0) acc *= -sctl[t].E;
                    tok_part[(((size_t)b * n_tiles + tile) * L + s + i0 + j) * 2 + col] = acc;
                }
            }
            if (WSYNC) wave_lds_sync(); else __syncthreads();
        }
    }
}

// One chunk of the backward replay, one workgroup per (chunk, 256 modes).
template <int K, int H, bool F32, bool FULL>
__device__ __forceinline__ void bwd_chunk(
    float (*lds)[64 * (2 * H + 1)], TokenCtl* sctl, const ModeConst& k, bool active, int lane, int wave,
    int tile, int n_tiles, int L, int M, int C, int b, int c, int mm, const TokenCtl* __restrict__ ctl,
    const uint32_t* __restrict__ drive, const float2* __restrict__ entries, const float2* __restrict__ mid,
    const uint32_t* __restrict__ dy, void* __restrict__ db, float* __restrict__ tok_part, cf& carry,
    float& acc_nu, float& acc_th) {
    constexpr int NH = K / H;
    const int s = c * K;
    const int kc = FULL ? K : min(K, L - s);
    const size_t row0 = ((size_t)b * L + s) * M;  // wave-uniform; the lane adds mm
    float4 tn = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((int)threadIdx.x < kc) tn = reinterpret_cast<const float4*>(ctl)[(size_t)b * L + s + threadIdx.x];
    cf ck[NH];
    uint32_t bw[K], gw[K];
    bwd_issue<K, H, FULL, false>(ck, bw, gw, kc, row0, M, mm, (size_t)b * C + c, entries, mid, drive, dy);
    if ((int)threadIdx.x < kc) reinterpret_cast<float4*>(sctl)[threadIdx.x] = tn;
    __syncthreads();
    bwd_body<K, H, F32, FULL, false>(lds[wave], sctl, k, active, lane, tile, n_tiles, L, M, b, s, kc, row0, mm, dy,
                                     db, tok_part, ck, bw, gw, carry, acc_nu, acc_th);
}

template <int K, int H, bool F32>
__global__ __launch_bounds__(BWD_THREADS) __attribute__((amdgpu_waves_per_eu(LRS_BWD_WAVES, 8))) void samu_bwd_replay_kernel(
    int L, int M, int C, int n_tiles, const TokenCtl* __restrict__ ctl,
    const uint32_t* __restrict__ drive, const float4* __restrict__ mtab,
    const float2* __restrict__ entries, const float2* __restrict__ mid, const float2* __restrict__ carry_in,
    const uint32_t* __restrict__ dy, void* __restrict__ db, float2* __restrict__ dz0,
    float* __restrict__ tok_part, float2* __restrict__ mode_part) {
    static_assert(K % H == 0 && 64 % (2 * H) == 0, "sub-chunk shape");
    __shared__ float lds[BWD_THREADS / 64][64 * (2 * H + 1)];
    __shared__ TokenCtl sctl[K];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = blockIdx.x * BWD_THREADS + threadIdx.x;
    const int c = blockIdx.y, b = blockIdx.z;
    const bool active = m < M;
    const int mm = active ? m : M - 1;
    const ModeConst k = load_mode(mtab, mm);
    const int tile = blockIdx.x * (BWD_THREADS / 64) + wave;
    const size_t cidx = ((size_t)b * C + c) * M + mm;
    const float2 ci = carry_in[cidx];
    cf carry = {ci.x, ci.y};
    float acc_nu = 0.f, acc_th = 0.f;
    // full chunks of workgroups whose lanes all hold a mode take a copy with
    // the per-token lane masks folded away
    if ((c + 1) * K <= L && (int)(blockIdx.x + 1) * BWD_THREADS <= M)
        bwd_chunk<K, H, F32, true>(lds, sctl, k, true, lane, wave, tile, n_tiles, L, M, C, b, c, mm, ctl,
                                   drive, entries, mid, dy, db, tok_part, carry, acc_nu, acc_th);
    else if ((c + 1) * K <= L)
        bwd_chunk<K, H, F32, true>(lds, sctl, k, active, lane, wave, tile, n_tiles, L, M, C, b, c, mm, ctl,
                                   drive, entries, mid, dy, db, tok_part, carry, acc_nu, acc_th);
    else
        bwd_chunk<K, H, F32, false>(lds, sctl, k, active, lane, wave, tile, n_tiles, L, M, C, b, c, mm, ctl,
                                    drive, entries, mid, dy, db, tok_part, carry, acc_nu, acc_th);
    if (active) {
        mode_part[cidx] = make_float2(-acc_nu, acc_th);
        if (dz0 && c == 0) dz0[(size_t)b * M + mm] = make_float2(carry.re, carry.im);
    }
}

constexpr int GB_LANES = 64;
// Tokens per partial-sum transpose in the single-pass backward: 8 when the
// chunk has earlier sub-chunks, whose cotangent words then take the LDS the
// smaller rows leave free, else the sub-chunk.
__host__ __device__ constexpr inline int gb_row_tokens(int K, int H) { return K > H ? 8 : H; }

// Single-pass grouped backward: the reverse summaries, the carry entering
// each group and the backward replay in one launch.  A workgroup owns one
// group of G chunks in the adjoint's processing order (wave w on chunk
// C - 1 - (q G + w)) and 64 modes.  Each wave reads its chunk's cotangent
// words once for the conjugate reverse summary (and keeps the last
// sub-chunk's words for the replay) and puts the chunk's map into the
// group's LDS table; the carry entering the group comes from the groups after
// it in time through group_handoff (the fixed-order chain of common.hpp,
// seeded with dz_final); wave w then applies the group's earlier maps to it
// to get the cotangent arriving after its chunk, and runs the adjoint of its
// chunk (bwd_body) with wave-local LDS traffic only.  The reverse summaries
// and group carries never go to memory as tensors.
template <int K, int H, bool F32, bool ALLACT>
__device__ __forceinline__ void gbscan_body(float4* gdyn, int G, int L, int M, int C, int n_tiles,
                                            const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
                                            const float4* __restrict__ mtab, const float2* __restrict__ entries,
                                            const float2* __restrict__ mid, const float4* __restrict__ chunk_rec,
                                            const float2* __restrict__ dz_final, uint64_t* __restrict__ pub,
                                            const uint32_t* __restrict__ dy, void* __restrict__ db,
                                            float2* __restrict__ dz0, float* __restrict__ tok_part,
                                            float2* __restrict__ mode_part, int polls) {
    constexpr int NH = K / H;
    constexpr int KE = K - H;  // tokens of the earlier sub-chunks
    constexpr int RH = gb_row_tokens(K, H);
    constexpr int ROW = 64 * (2 * RH + 1);  // floats of one wave's transpose rows
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    // LDS: [G][64] entry states, [G][K] token controls, [G][KE][64] the
    // earlier sub-chunks' cotangent words, [G][ROW] transpose rows; the
    // group's summary table and the hand-off scratch ([G][64] float4 each)
    // overlay the rows (read only before the last barrier ahead of the
    // replay, the rows only after it)
    float2* stash = reinterpret_cast<float2*>(gdyn) + w * GB_LANES + lane;
    TokenCtl* sctl = reinterpret_cast<TokenCtl*>(reinterpret_cast<float2*>(gdyn) + G * GB_LANES) + w * K;
    uint32_t* dys = reinterpret_cast<uint32_t*>(reinterpret_cast<TokenCtl*>(reinterpret_cast<float2*>(gdyn) +
                                                                             G * GB_LANES) + G * K);
    float* rows = reinterpret_cast<float*>(dys + G * KE * 64);
    uint32_t* dy_w = dys + w * KE * 64 + lane;
    float* lds_w = rows + w * ROW;
    float4* comp = reinterpret_cast<float4*>(rows);
    float4* look = comp + G * GB_LANES;
    const int q = blockIdx.y, b = blockIdx.z, NG = gridDim.y;
    const int pc = q * G + w;
    const bool valid = pc < C;  // wave-uniform
    const int c = C - 1 - min(pc, C - 1);
    const int m = blockIdx.x * GB_LANES + lane;
    const bool active = ALLACT || m < M;
    const int mm = active ? m : M - 1;
    const int tile = blockIdx.x;
    const int s = c * K;
    const int kc = min(K, L - s);
    const size_t row0 = ((size_t)b * L + s) * M;  // wave-uniform
    const size_t bc = (size_t)b * C + c;

    // requests: token controls, mode constants, the chunk record, every
    // cotangent word of the chunk (last token first, the order the reverse
    // summary takes them in; past a partial chunk's end they read as 0),
    // then the replay's states and drive words.  The drive and cotangent
    // words are read once here and by no later kernel of the step, so they
    // carry the non-temporal hint.
    float4 tn = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < kc) tn = reinterpret_cast<const float4*>(ctl)[(size_t)b * L + s + lane];
    const ModeConst k = load_mode(mtab, mm);
    const float4 ph = mtab[MODE_REC * mm + (c == C - 1 ? 3 : 2)];
    const float4 rec = chunk_rec[bc];
    // the replay's requests as the grouped replay makes them (its states, all
    // drive words, the last sub-chunk's cotangent words), then the earlier
    // sub-chunks' cotangent words, which only the summary uses here (the
    // replay requests them again as their sub-chunk starts)
    cf ck[NH];
    uint32_t bw[K], gw[K];
    bwd_issue<K, H, false, true>(ck, bw, gw, kc, row0, M, mm, bc, entries, mid, drive, dy);
    uint32_t ge[KE > 0 ? KE : 1];
    if (KE > 0) {
        const ChunkRows cr(dy + row0, kc, M);
#pragma unroll
        for (int j = 0; j < KE; ++j) ge[KE - 1 - j] = cr.load_nt(KE - 1 - j, mm);
    }
    if (lane < kc) reinterpret_cast<float4*>(sctl)[lane] = tn;
    wave_lds_sync();
    // the controls through one vector-register base kept for the whole chunk
    // (an LDS read needs its address in a vector register)
    const TokenCtl* sv = sctl + opaque_v(0u);
    // the chunk's conjugate reverse summary: carry -> conj(lambda_t) (dy_t + carry)
    cf A = {1.f, 0.f}, Bv = {0.f, 0.f};
    if (valid) {
        const int kq = opaque(kc);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int i = K - 1 - j;
            if (i < kq) {
                const TokenCtl t = sv[i];
                const cf lam = mode_lambda(k, t.E, t.C, t.S);
                const uint32_t x = i >= KE ? gw[i] : ge[i < KE ? i : 0];
                Bv = cmulc(lam, {Bv.re + bf16_lo(x), Bv.im + bf16_hi(x)});
            }
        }
        A = chunk_transition<true>(k.kappa, ph, rec);
    }
    // the earlier sub-chunks' words wait in LDS for the replay
#pragma unroll
    for (int i = 0; i < KE; ++i) dy_w[i * 64] = ge[i];
    comp[w * GB_LANES + lane] = make_float4(A.re, A.im, Bv.re, Bv.im);
    if (NH > 1) *stash = make_float2(ck[0].re, ck[0].im);
    __syncthreads();
    // the cotangent entering the group, then the one arriving after this
    // chunk: the group's earlier summaries (processing order) applied to it
    const GroupChunks gc{chunk_rec + (size_t)b * C, mtab[MODE_REC * mm + 2], mtab[MODE_REC * mm + 3], k.kappa, C};
    const float4 gin = group_handoff<true>(comp, look, G, w, lane, q, NG, M, mm, active,
                                           dz_final ? dz_final + (size_t)b * M : nullptr,
                                           pub + (size_t)b * NG * SCAN_PUB_WORDS * M, gc, polls);
    cf carry = {gin.x, gin.y};
    if (valid) {
        for (int j = 0; j < w; ++j) {
            const float4 f = comp[j * GB_LANES + lane];
            carry = cfma({f.x, f.y}, carry, {f.z, f.w});
        }
    }
    __syncthreads();  // the summary table's LDS becomes the transpose rows
    float acc_nu = 0.f, acc_th = 0.f;
    if (valid) {
        // the last sub-chunk's cotangent words are still held from the
        // summary, the earlier sub-chunks' wait in LDS
        bwd_body<K, H, F32, false, true, true, (NH > 1), RH, (KE > 0), !F32>(
            lds_w, sv, k, active, lane, tile, n_tiles, L, M, b, s, kc, row0, mm, dy, db, tok_part, ck, bw, gw,
            carry, acc_nu, acc_th, stash, dy_w);
        if (active && dz0 && c == 0) dz0[(size_t)b * M + m] = make_float2(carry.re, carry.im);
    }
    // the (d nu, d theta) partials of the group's chunks, added in processing
    // order through the waves' stash slots (free again): one row per group
    *stash = make_float2(-acc_nu, acc_th);
    __syncthreads();
    if (w == 0 && active) {
        const float2* part = reinterpret_cast<const float2*>(gdyn) + lane;
        const int n = min(G, C - q * G);
        float sx = 0.f, sy = 0.f;
        for (int j = 0; j < n; ++j) {
            const float2 v = part[j * GB_LANES];
            sx += v.x;
            sy += v.y;
        }
        mode_part[((size_t)b * NG + q) * M + m] = make_float2(sx, sy);
    }
}

template <int K, int H, bool F32>
__global__ __launch_bounds__(GB_LANES * SAMU_GROUP_MAX) __attribute__((amdgpu_waves_per_eu(4, 8))) void
samu_gbscan_kernel(int L, int M, int C, int G, int n_tiles, const TokenCtl* __restrict__ ctl,
                   const uint32_t* __restrict__ drive, const float4* __restrict__ mtab,
                   const float2* __restrict__ entries, const float2* __restrict__ mid,
                   const float4* __restrict__ chunk_rec, const float2* __restrict__ dz_final,
                   uint64_t* __restrict__ pub, const uint32_t* __restrict__ dy, void* __restrict__ db,
                   float2* __restrict__ dz0, float* __restrict__ tok_part, float2* __restrict__ mode_part,
                   int polls) {
    static_assert(K % H == 0 && 64 % (2 * H) == 0, "sub-chunk shape");
    extern __shared__ float4 gdyn[];
    if ((int)(blockIdx.x + 1) * GB_LANES <= M)  // uniform over the workgroup
        gbscan_body<K, H, F32, true>(gdyn, G, L, M, C, n_tiles, ctl, drive, mtab, entries, mid, chunk_rec, dz_final,
                                     pub, dy, db, dz0, tok_part, mode_part, polls);
    else
        gbscan_body<K, H, F32, false>(gdyn, G, L, M, C, n_tiles, ctl, drive, mtab, entries, mid, chunk_rec,
                                      dz_final, pub, dy, db, dz0, tok_part, mode_part, polls);
}

// Zeroes n 16-byte words (the single-pass backward's hand-off area, before
// the pass).
__global__ __launch_bounds__(256) void clear_words_kernel(uint4* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// -------------------------------------------------- controller backward ---
// One workgroup per block of CTL_TB tokens; threads own 8 selector columns at
// a time.  The second stage of the shared-control reduction (over the mode
// tiles, fixed order) happens here, then p-bar, r-bar and the per-token u-bar
// follow; dx_sel = u-bar_phi w^_phi + u-bar_r w^_r.  The block writes its
// partial sums of u-bar * x~ for every column of x~ plus three scalar pairs:
//   column D     sum u-bar            (the constant 1 of x~)
//   column D+1   sum d-bar p, sum c-bar q       (amplitude gradients)
//   column D+2   sum u-bar u  with u = x~ . w^  (= w^ . g, for the projection)
constexpr int CTL_TB = 64;
// dx_sel stores carry the non-temporal hint like the other output streams
// (measured: a plain store makes this kernel faster but the pass slower, as
// the next kernel then writes the dirty lines back)
#ifndef LRS_DX_NT
#define LRS_DX_NT 1
#endif
constexpr bool DX_NT = LRS_DX_NT != 0;

// Threads: CT column threads (16-byte column groups) x TS token splits of the
// block's CTL_TB tokens; the TS partial sums of u-bar * x~ of a column group
// are added in split order through LDS, so the result is fixed for a given D.
constexpr int CTL_TOKB = 16;  // tokens whose selector words are loaded together

// Token tok0 + i clamped to the last token (unsigned: tok0 + i may pass 2^31 - 1).
__device__ __forceinline__ int clamp_tok(int tok0, int i, int BL) {
    return (int)min((unsigned)tok0 + (unsigned)i, (unsigned)(BL - 1));
}

// Selector words of tokens tok0 .. tok0 + CTL_TOKB - 1 in column group j8.
// Tokens are clamped into the tensor, so every load is issued unconditionally
// (a guarded load becomes a branch, after which waiting for any earlier
// request turns into waiting for all of them); the consumer skips the rest.
// This is the step's last read of x_sel, so the loads carry the non-temporal
// hint.
__device__ __forceinline__ void ctl_load_batch(uint4 (&xv)[CTL_TOKB], const uint4* __restrict__ x_sel, int tok0,
                                               int BL, int D8, int j8) {
#pragma unroll
    for (int t = 0; t < CTL_TOKB; ++t) {
        const uint4* row = x_sel + (size_t)clamp_tok(tok0, t, BL) * D8;  // wave-uniform
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(&row[j8]));
        xv[t] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// Tile partials of a block staged through LDS (the first wave reads any
// further ones directly), and how many each thread requests up front.
constexpr int CTL_LDS_TILES = 64;
constexpr int CTL_TPL = 2;

template <bool F32>
__global__ __launch_bounds__(1024) void samu_ctl_bwd_kernel(
    int B, int L, int D, int M, int n_tiles, int TS, const uint4* __restrict__ x_sel,
    const float* __restrict__ w_phi, const float* __restrict__ w_r,
    const float* __restrict__ a_phi, const float* __restrict__ a_r,
    const float* __restrict__ p_sv, const float* __restrict__ r_sv,
    const float2* __restrict__ u_sv, const float* __restrict__ inv_norm, const float* __restrict__ tok_part,
    void* __restrict__ dx, float* __restrict__ g_part) {
    // the block's tile partials [tiles][CTL_TB] float2, later the split sums [TS - 1][4][CT]
    extern __shared__ float4 dyn[];
    float4* comb = dyn;
    __shared__ float u_sh[2][CTL_TB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nthr = blockDim.x;
    const int BL = B * L;
    const int blk = blockIdx.x;
    const int ncol = D + 4;
    const int D8 = D >> 3;
    const int CT = blockDim.x / TS;
    // CT is a multiple of 64, so a wave lies in one split: make that visible
    // to the compiler, and every token row offset becomes a scalar
    const int ts = __builtin_amdgcn_readfirstlane(tid / CT), cj = tid - ts * CT;
    const int ntok = min(CTL_TB, BL - blk * CTL_TB);
    const int tper = CTL_TB / TS;
    const int tlo = ts * tper, thi = min(tlo + tper, ntok);
    const size_t tokb = (size_t)blk * CTL_TB;
    const int tokb32 = blk * CTL_TB;

    // Requests that do not wait on the selector stream go first, so the
    // first wave forms u-bar while the selector words are in flight: the
    // block's tile partials (coalesced over tokens) and the per-token saved
    // values of the first wave's tokens.
    const int ltiles = min(n_tiles, CTL_LDS_TILES);
    const int npairs = ltiles * CTL_TB;
    const float2* tp2 = reinterpret_cast<const float2*>(tok_part);
    float2 tv[CTL_TPL];
#pragma unroll
    for (int k = 0; k < CTL_TPL; ++k) {
        const int idx = min(tid + k * nthr, npairs - 1);
        const int tok = clamp_tok(tokb32, idx % CTL_TB, BL);
        const int bb = tok / L;
        tv[k] = tp2[((size_t)bb * n_tiles + idx / CTL_TB) * L + (tok - bb * L)];
    }
    const int mytok = clamp_tok(tokb32, lane, BL);
    const float pv = p_sv[mytok], rv = r_sv[mytok];
    const float2 uv = u_sv[mytok];

    // the first selector batch
    uint4 xv[CTL_TOKB];
    ctl_load_batch(xv, x_sel, tokb32 + tlo, BL, D8, min(cj, D8 - 1));
    __builtin_amdgcn_sched_barrier(0);

    // per-token u-bar: the tiles summed in order by the first wave (CTL_TB == 64)
    float2* tps = reinterpret_cast<float2*>(dyn);
#pragma unroll
    for (int k = 0; k < CTL_TPL; ++k) tps[min(tid + k * nthr, npairs - 1)] = tv[k];  // repeats store equal values
    for (int idx = CTL_TPL * nthr + tid; idx < npairs; idx += nthr) {
        const int tok = clamp_tok(tokb32, idx % CTL_TB, BL);
        const int bb = tok / L;
        tps[idx] = tp2[((size_t)bb * n_tiles + idx / CTL_TB) * L + (tok - bb * L)];
    }
    __syncthreads();
    if (wave == 0) {
        const bool valid = lane < ntok;
        float cb = 0.f, dbr = 0.f;
        for (int t = 0; t < ltiles; ++t) {
            const float2 v = tps[t * CTL_TB + lane];
            cb += v.x;
            dbr += v.y;
        }
        if (n_tiles > ltiles) {  // tiles beyond the staged ones, in order
            const int bb = mytok / L;
            const float2* tq = tp2 + (size_t)bb * n_tiles * L + (mytok - bb * L);
            for (int t = ltiles; t < n_tiles; ++t) {
                const float2 v = tq[(size_t)t * L];
                cb += v.x;
                dbr += v.y;
            }
        }
        const float r2 = rv * rv;
        const float q = rv / (1.0f + r2);
        const float sM = sqrtf((float)M);
        const float pbar = dbr * tanhf(a_phi[0]) / sM;
        const float rbar = cb * tanhf(a_r[0]) / sM * (1.0f - r2) / ((1.0f + r2) * (1.0f + r2));
        const float uphi = valid ? pbar * (1.0f - pv * pv) : 0.f;
        const float ur = valid ? rbar * (1.0f - r2) : 0.f;
        const float sdp = valid ? dbr * pv : 0.f;
        const float scq = valid ? cb * q : 0.f;
        u_sh[0][lane] = uphi;
        u_sh[1][lane] = ur;
        const float s0 = wave_sum(uphi), s1 = wave_sum(ur), s2 = wave_sum(sdp), s3 = wave_sum(scq);
        const float s4 = wave_sum(uphi * uv.x), s5 = wave_sum(ur * uv.y);
        if (lane == 0) {
            float4* gq = reinterpret_cast<float4*>(g_part + ((size_t)blk * ncol + D) * 2);
            gq[0] = make_float4(s0, s1, s2, s3);
            gq[1] = make_float4(s4, s5, 0.f, 0.f);
        }
    }
    __syncthreads();
    // 1/||w||, kept by the forward controller
    const float inv_phi = inv_norm[0], inv_r = inv_norm[1];

    for (int jb = 0; jb < D8; jb += CT) {  // uniform trip count: barriers below
        const int j8 = jb + cj;
        const bool act = j8 < D8;
        float wp[8], wr[8], gp[8], gr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { wp[e] = 0.f; wr[e] = 0.f; gp[e] = 0.f; gr[e] = 0.f; }
        if (act) {
            const float4* a = reinterpret_cast<const float4*>(w_phi) + 2 * j8;
            const float4* c = reinterpret_cast<const float4*>(w_r) + 2 * j8;
            const float4 a0 = a[0], a1 = a[1], c0 = c[0], c1 = c[1];
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wp[e] = av[e] * inv_phi;
                wr[e] = cv[e] * inv_r;
            }
        }
        for (int t0 = tlo; t0 < thi; t0 += CTL_TOKB) {
            const int nt = min(CTL_TOKB, thi - t0);
            if (jb > 0 || t0 > tlo) ctl_load_batch(xv, x_sel, tokb32 + t0, BL, D8, min(j8, D8 - 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < CTL_TOKB; ++t) {
                if (t >= nt) continue;  // no early exit: the loop must unroll
                const size_t tok = tokb + t0 + t;
                const float uphi = u_sh[0][t0 + t], ur = u_sh[1][t0 + t];
                const uint32_t xw[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
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
                if (act) {
                    if (F32) {
                        float4* row = reinterpret_cast<float4*>(dx) + tok * D8 * 2;  // wave-uniform
                        out_store<f32x4_t, DX_NT>(row + 2 * j8, f32x4_t{o[0], o[1], o[2], o[3]});
                        out_store<f32x4_t, DX_NT>(row + 2 * j8 + 1, f32x4_t{o[4], o[5], o[6], o[7]});
                    } else {
                        uint4* row = reinterpret_cast<uint4*>(dx) + tok * D8;  // wave-uniform
                        out_store<u32x4_t, DX_NT>(row + j8, u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                                    pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])});
                    }
                }
            }
        }
        // partial sums of the token splits, added in split order
        if (TS > 1) {
            if (act && ts > 0) {
                // [split][quarter][column thread]: lanes write adjacent 16-byte words
                float4* c = comb + (size_t)(ts - 1) * 4 * CT + cj;
                c[0] = make_float4(gp[0], gp[1], gp[2], gp[3]);
                c[CT] = make_float4(gp[4], gp[5], gp[6], gp[7]);
                c[2 * CT] = make_float4(gr[0], gr[1], gr[2], gr[3]);
                c[3 * CT] = make_float4(gr[4], gr[5], gr[6], gr[7]);
            }
            __syncthreads();
            if (act && ts == 0) {
                for (int k = 1; k < TS; ++k) {
                    const float4* c = comb + (size_t)(k - 1) * 4 * CT + cj;
                    const float4 c0 = c[0], c1 = c[CT], c2 = c[2 * CT], c3 = c[3 * CT];
                    gp[0] += c0.x; gp[1] += c0.y; gp[2] += c0.z; gp[3] += c0.w;
                    gp[4] += c1.x; gp[5] += c1.y; gp[6] += c1.z; gp[7] += c1.w;
                    gr[0] += c2.x; gr[1] += c2.y; gr[2] += c2.z; gr[3] += c2.w;
                    gr[4] += c3.x; gr[5] += c3.y; gr[6] += c3.z; gr[7] += c3.w;
                }
            }
            __syncthreads();
        }
        if (act && ts == 0) {
            float4* out = reinterpret_cast<float4*>(g_part + ((size_t)blk * ncol + 8 * j8) * 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = make_float4(gp[2 * e], gr[2 * e], gp[2 * e + 1], gr[2 * e + 1]);
        }
    }
}

// ------------------------------------------------ parameter reductions ---
// One launch sums the token-block partials g_part [n_blk, D+4] (a float2 of
// phi and r terms per column) and the chunk (or group) partials mode_part
// [mode_rows, M] (a
// float2 of nu and theta terms per mode) in FP64 and in a fixed order, then
// forms the parameter gradients.  A workgroup owns PR_ITEMS columns (or
// modes) and splits the rows over PR_SG thread groups: group sg adds rows
// sg, sg + PR_SG, ... in order, PR_NB of them requested at once, and the
// group sums are added in group order through LDS, PR_L2 at a time.  The
// result depends on the shape alone.  Column workgroups also form the sums
// of the scalar columns and, with the FP64 squared direction norms the
// forward controller kept,
// dw = (g - w^ (w^ . g)) / ||w|| with w^ . g from the per-token sums of
// u-bar * u (column D+2); the first one also writes da from column D+1.
// A few MB in all, so the layout aims at few dependent rounds of loads with
// one 1024-thread workgroup per CU.  (Issuing the scalar-column and row loads
// of a column workgroup together measured slower than this order.)
constexpr int PR_ITEMS = 16;
constexpr int PR_SG = 64;
constexpr int PR_THREADS = PR_ITEMS * PR_SG;
constexpr int PR_NB = 16;
constexpr int PR_L2 = 8;
constexpr int PR_NORM = 4;  // direction entries per thread per round of loads

struct ParamLds {
    double2 g1[PR_SG][PR_ITEMS];
    double2 g2[PR_SG / PR_L2][PR_ITEMS];
    double2 scal[2];
};

// Sum of item `item` over rows [0, n) of part (row stride `stride`); valid in
// the threads with sg == 0.
__device__ __forceinline__ double2 pr_rows_sum(const float2* __restrict__ part, size_t stride, int item, int n,
                                               int sg, int ii, ParamLds& sh) {
    double sx = 0.0, sy = 0.0;
    for (int r0 = sg; r0 < n; r0 += PR_SG * PR_NB) {
        float2 v[PR_NB];
#pragma unroll
        for (int k = 0; k < PR_NB; ++k) v[k] = part[(size_t)min(r0 + k * PR_SG, n - 1) * stride + item];
#pragma unroll
        for (int k = 0; k < PR_NB; ++k) {
            const bool ok = r0 + k * PR_SG < n;
            sx += ok ? (double)v[k].x : 0.0;
            sy += ok ? (double)v[k].y : 0.0;
        }
    }
    sh.g1[sg][ii] = make_double2(sx, sy);
    __syncthreads();
    if (sg < PR_SG / PR_L2) {
        double tx = 0.0, ty = 0.0;
#pragma unroll
        for (int g = 0; g < PR_L2; ++g) {
            tx += sh.g1[sg * PR_L2 + g][ii].x;
            ty += sh.g1[sg * PR_L2 + g][ii].y;
        }
        sh.g2[sg][ii] = make_double2(tx, ty);
    }
    __syncthreads();
    double tx = 0.0, ty = 0.0;
    if (sg == 0) {
#pragma unroll
        for (int g = 0; g < PR_SG / PR_L2; ++g) {
            tx += sh.g2[g][ii].x;
            ty += sh.g2[g][ii].y;
        }
    }
    return make_double2(tx, ty);
}

__global__ __launch_bounds__(PR_THREADS) void samu_param_kernel(
    int D, int M, int col_blocks, const float* __restrict__ w_phi, const float* __restrict__ w_r,
    const float* __restrict__ a_phi, const float* __restrict__ a_r, const double* __restrict__ wnorm2,
    const float2* __restrict__ g_part, int n_blk, const float2* __restrict__ mode_part, int nchunks,
    float* __restrict__ dw_phi, float* __restrict__ dw_r,
    float* __restrict__ da_phi, float* __restrict__ da_r, float* __restrict__ dnu, float* __restrict__ dtheta) {
    __shared__ ParamLds sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sg = tid / PR_ITEMS, ii = tid - sg * PR_ITEMS;
    if ((int)blockIdx.x >= col_blocks) {
        const int m0 = (blockIdx.x - col_blocks) * PR_ITEMS;
        const int m = min(m0 + ii, M - 1);
        const double2 t = pr_rows_sum(mode_part, M, m, nchunks, sg, ii, sh);
        if (sg == 0 && m0 + ii < M) {
            dnu[m] = (float)t.x;
            dtheta[m] = (float)t.y;
        }
        return;
    }
    const int ncol = D + 4;
    const int j = min((int)blockIdx.x * PR_ITEMS + ii, D);
    const float wpj = w_phi[j], wrj = w_r[j];
    // FP64 squared direction norms, formed by the forward controller
    const double Np = wnorm2[0], Nr = wnorm2[1];
    // the scalar columns D+1 and D+2 over all token blocks: rows lane,
    // lane + 64, ... of the first wave, then a fixed butterfly
    if (wave == 0) {
        double s1x = 0.0, s1y = 0.0, s2x = 0.0, s2y = 0.0;
        for (int r0 = lane; r0 < n_blk; r0 += 64 * PR_NB) {
            float2 v1[PR_NB], v2[PR_NB];
#pragma unroll
            for (int k = 0; k < PR_NB; ++k) {
                const size_t row = (size_t)min(r0 + k * 64, n_blk - 1) * ncol;
                v1[k] = g_part[row + D + 1];
                v2[k] = g_part[row + D + 2];
            }
#pragma unroll
            for (int k = 0; k < PR_NB; ++k) {
                const bool ok = r0 + k * 64 < n_blk;
                s1x += ok ? (double)v1[k].x : 0.0;
                s1y += ok ? (double)v1[k].y : 0.0;
                s2x += ok ? (double)v2[k].x : 0.0;
                s2y += ok ? (double)v2[k].y : 0.0;
            }
        }
        s1x = wave_sum_d(s1x);
        s1y = wave_sum_d(s1y);
        s2x = wave_sum_d(s2x);
        s2y = wave_sum_d(s2y);
        if (lane == 0) {
            sh.scal[0] = make_double2(s1x, s1y);  // sum d-bar p, sum c-bar q
            sh.scal[1] = make_double2(s2x, s2y);  // w^ . g for phi and r
        }
    }
    const double2 g = pr_rows_sum(g_part, ncol, j, n_blk, sg, ii, sh);  // its barriers cover scal
    if (sg != 0 || (int)blockIdx.x * PR_ITEMS + ii > D) return;
    const double np = sqrt(Np), nrr = sqrt(Nr);
    const double2 dot = sh.scal[1];
    dw_phi[j] = (float)((g.x - ((double)wpj / np) * dot.x) / np);
    dw_r[j] = (float)((g.y - ((double)wrj / nrr) * dot.y) / nrr);
    if (j == 0) {
        const double2 sa = sh.scal[0];
        const double sM = sqrt((double)M);
        const double tp = tanh((double)a_phi[0]), tr = tanh((double)a_r[0]);
        da_phi[0] = (float)((1.0 - tp * tp) / sM * sa.x);
        da_r[0] = (float)((1.0 - tr * tr) / sM * sa.y);
    }
}

}  // namespace

int samu_bwd_tiles(int M) { return (int)ceil_div(M, 64); }
int samu_ctl_tok_per_blk() { return CTL_TB; }

hipError_t launch_samu_bwd_replay(const SamuParams& p, const Chunking& ch, const float* ctl,
                                  const float* mtab, const float* entries, const float* mid,
                                  const float* carry_in, const void* dy, void* db, int db_f32, float* dz0,
                                  float* tok_part, int n_tiles, float* mode_part, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(p.M, BWD_THREADS), ch.C, ch.B);
#define BWD_CASE(KK, HH, FF)                                                                             \
    LRS_LAUNCH(K_SAMU_BWD_REPLAY, (samu_bwd_replay_kernel<KK, HH, FF>), grid, dim3(BWD_THREADS), 0, s, \
               p.L, p.M, ch.C, n_tiles, (const TokenCtl*)ctl, (const uint32_t*)p.b,                   \
               (const float4*)mtab, (const float2*)entries, (const float2*)mid,                       \
               (const float2*)carry_in, (const uint32_t*)dy, db, (float2*)dz0, tok_part, (float2*)mode_part)
    constexpr int H32 = SAMU_BWD_SUB, H16 = SAMU_BWD_SUB < 16 ? SAMU_BWD_SUB : 16;
    if (ch.K == 32) {
        if (db_f32) BWD_CASE(32, H32, true); else BWD_CASE(32, H32, false);
    } else {
        if (db_f32) BWD_CASE(16, H16, true); else BWD_CASE(16, H16, false);
    }
#undef BWD_CASE
    return hipGetLastError();
}


hipError_t launch_clear_words(void* p, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div((int64_t)n16, 256), 2048));
    LRS_LAUNCH(K_CLEAR, clear_words_kernel, dim3(blocks), dim3(256), 0, s, (uint4*)p, n16);
    return hipGetLastError();
}

hipError_t launch_samu_gbscan(const SamuParams& p, const Chunking& ch, const float* ctl, const float* mtab,
                              const float* entries, const float* mid, const float* chunk_rec, const float* dz_final,
                              void* pub, size_t pub_bytes, const void* dy, void* db, int db_f32, float* dz0,
                              float* tok_part, int n_tiles, float* mode_part, hipStream_t s) {
    {
        const hipError_t e = launch_clear_words(pub, pub_bytes, s);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)ceil_div(p.M, GB_LANES), ch.NG, ch.B);
    const dim3 block(GB_LANES * ch.G);
    const int H = ch.K == 32 ? SAMU_BWD_SUB : 16;
    // entry-state stash, token controls, the earlier sub-chunks' cotangent
    // words, transpose rows (the summary table and the hand-off scratch
    // overlay the rows, which are larger)
    const size_t lds = (size_t)ch.G * GB_LANES * sizeof(float2) + (size_t)ch.G * ch.K * sizeof(TokenCtl) +
                       (size_t)ch.G * (ch.K - H) * 64 * sizeof(uint32_t) +
                       (size_t)ch.G * 64 * (2 * gb_row_tokens(ch.K, H) + 1) * sizeof(float);
#define GBSCAN_CASE(KK, HH, FF)                                                                            \
    LRS_LAUNCH(K_SAMU_BWD_SCAN, (samu_gbscan_kernel<KK, HH, FF>), grid, block, lds, s, p.L, p.M, ch.C, ch.G, \
               n_tiles, (const TokenCtl*)ctl, (const uint32_t*)p.b, (const float4*)mtab,                 \
               (const float2*)entries, (const float2*)mid, (const float4*)chunk_rec,                     \
               (const float2*)dz_final, (uint64_t*)pub, (const uint32_t*)dy, db, (float2*)dz0, tok_part, \
               (float2*)mode_part, handoff_poll_limit())
    constexpr int H32 = SAMU_BWD_SUB, H16 = SAMU_BWD_SUB < 16 ? SAMU_BWD_SUB : 16;
    if (ch.K == 32) {
        if (db_f32) GBSCAN_CASE(32, H32, true); else GBSCAN_CASE(32, H32, false);
    } else {
        if (db_f32) GBSCAN_CASE(16, H16, true); else GBSCAN_CASE(16, H16, false);
    }
#undef GBSCAN_CASE
    return hipGetLastError();
}

hipError_t launch_samu_ctl_bwd(const SamuParams& p, const float* p_sv, const float* r_sv,
                               const float* u_sv, const float* inv_norm, const float* tok_part, int n_tiles,
                               void* dx_sel, int dx_f32, float* g_part, hipStream_t s) {
    const int BL = p.B * p.L;
    const int grid = (int)ceil_div(BL, CTL_TB);
    // column threads (a multiple of 64, at most 1024) and token splits (1, 2 or 4)
    const int CT = (int)std::min<int64_t>(1024, ceil_div(p.D / 8, 64) * 64);
    int TS = 1;
    while (TS < 4 && CT * TS * 2 <= 1024) TS *= 2;
    const size_t shmem = std::max((size_t)(TS - 1) * CT * 4 * sizeof(float4),
                                  (size_t)std::min(n_tiles, CTL_LDS_TILES) * CTL_TB * sizeof(float2));
#define CTLB_CASE(FF)                                                                                    \
    LRS_LAUNCH(K_SAMU_CTL_BWD, samu_ctl_bwd_kernel<FF>, dim3(grid), dim3(CT * TS), shmem, s, p.B, p.L, p.D, \
               p.M, n_tiles, TS, (const uint4*)p.x_sel, p.w_phi, p.w_r, p.a_phi, p.a_r, p_sv, r_sv,        \
               (const float2*)u_sv, inv_norm, tok_part, dx_sel, g_part)
    if (dx_f32) CTLB_CASE(true); else CTLB_CASE(false);
#undef CTLB_CASE
    return hipGetLastError();
}

int samu_param_columns(int D) { return D + 4; }

hipError_t launch_samu_params(const SamuParams& p, const Chunking& ch, const double* wnorm2, const float* g_part,
                              int n_blk, const float* mode_part, int mode_rows, float* dw_phi, float* dw_r,
                              float* da_phi, float* da_r, float* dnu, float* dtheta, hipStream_t s) {
    const int col_blocks = (int)ceil_div(p.D + 1, PR_ITEMS);
    const int grid = col_blocks + (int)ceil_div(p.M, PR_ITEMS);
    LRS_LAUNCH(K_SAMU_PARAMS, samu_param_kernel, dim3(grid), dim3(PR_THREADS), 0, s, p.D, p.M, col_blocks,
               p.w_phi, p.w_r, p.a_phi, p.a_r, wnorm2, (const float2*)g_part, n_blk, (const float2*)mode_part,
               mode_rows, dw_phi, dw_r, da_phi, da_r, dnu, dtheta);
    return hipGetLastError();
}

}  // namespace lrs
