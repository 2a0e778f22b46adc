// gate_proj.hip -- the RG-LRU gate projections on MFMA: two 16-block
// block-diagonal linear layers in front of the gated scan, and their adjoint.
//
// Page 'Griffin 第 4、5 节 H800 对照协议', 'RG-LRU 的固定方程': both gates are
// computed by 16-block block-diagonal linear layers; training runs them in
// BF16 autocast.  With Db = D/16 and block i covering channels
// [i Db, (i+1) Db), weights stored [16, Db, Db] as (block, output, input):
//   l[t, i Db + o] = b[i Db + o] + sum_k W[i][o][k] x[t, i Db + k]
// for l = l^x (W_x, b_x) and l = l^a (W_a, b_a), rounded to BF16 for the scan.
// Adjoint for the logit cotangents dl^x, dl^a produced by the scan backward:
//   dx[t, i Db + k] += sum_o (W_x[i][o][k] dl^x + W_a[i][o][k] dl^a)[t, i Db + o]
//   dW[i][o][k] = sum_t dl[t, i Db + o] x[t, i Db + k],  db = sum_t dl.
//
// Matrix-core layout (v_mfma_f32_16x16x16_bf16; 16x16x4_f32 for FP32
// cotangents): lane l holds A[l%16][4(l/16)+j] and B[4(l/16)+j][l%16],
// j = 0..3, and receives D[4(l/16)+r][l%16], r = 0..3.  Every product is
// arranged so that D's rows run over channels and its columns over tokens:
// each lane then owns four consecutive channels of one token, one 8- or
// 16-byte store.  Tiles are staged in LDS with rows padded by 4 elements so
// the 16 rows a fragment read touches fall on different banks.
#include "common.hpp"

namespace lrs {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int GP_THREADS = 256;   // 4 waves
constexpr int GP_TT = 64;         // tokens per workgroup in the forward and dx kernels
constexpr int GP_PAD = 4;         // elements of padding per LDS row
constexpr int GP_RANGE = 2048;    // tokens per dW partial

__device__ __forceinline__ v4s lds4(const uint16_t* p) { return *reinterpret_cast<const v4s*>(p); }

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) { return pack_bf16x2(lo, hi); }

// Copy a [rows, Db] BF16 tile (row stride `gstride` elements) into LDS rows of
// Db + GP_PAD elements, 16 bytes per thread step; rows past `valid` are zero.
__device__ __forceinline__ void stage_rows(uint16_t* lds, const uint16_t* g, size_t gstride, int rows, int valid,
                                           int Db) {
    const int per_row = Db / 8;
    for (int c = threadIdx.x; c < rows * per_row; c += GP_THREADS) {
        const int r = c / per_row, k8 = (c - r * per_row) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < valid) v = *reinterpret_cast<const uint4*>(g + (size_t)r * gstride + k8);
        uint16_t* d = lds + r * (Db + GP_PAD) + k8;
        reinterpret_cast<uint2*>(d)[0] = make_uint2(v.x, v.y);
        reinterpret_cast<uint2*>(d)[1] = make_uint2(v.z, v.w);
    }
}

// ------------------------------------------------------------- forward ---
// grid (ceil(BL / GP_TT), 16 blocks); wave w owns tokens [16 w, 16 w + 16).
__global__ __launch_bounds__(GP_THREADS) void gate_proj_fwd_kernel(
    int BL, int D, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_x,
    const float* __restrict__ b_x, const uint16_t* __restrict__ w_a, const float* __restrict__ b_a,
    uint16_t* __restrict__ lx, uint16_t* __restrict__ la) {
    extern __shared__ uint16_t gp_lds[];
    const int Db = D / 16, RS = Db + GP_PAD;
    uint16_t* sWx = gp_lds;
    uint16_t* sWa = sWx + Db * RS;
    uint16_t* sX = sWa + Db * RS;
    const int blk = blockIdx.y;
    const size_t t0 = (size_t)blockIdx.x * GP_TT;
    const int valid = (int)min((size_t)GP_TT, (size_t)BL - t0);
    stage_rows(sWx, w_x + (size_t)blk * Db * Db, Db, Db, Db, Db);
    stage_rows(sWa, w_a + (size_t)blk * Db * Db, Db, Db, Db, Db);
    stage_rows(sX, x + t0 * D + (size_t)blk * Db, D, GP_TT, valid, Db);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int MT = Db / 16;
    const uint16_t* xrow = sX + (wave * 16 + col) * RS + 4 * grp;  // B = x^T, token column `col`
    for (int mt = 0; mt < MT; ++mt) {
        v4f ax = {0.f, 0.f, 0.f, 0.f}, aa = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* wxr = sWx + (mt * 16 + col) * RS + 4 * grp;  // A = W rows (outputs)
        const uint16_t* war = sWa + (mt * 16 + col) * RS + 4 * grp;
        for (int kb = 0; kb < Db; kb += 16) {
            const v4s bx = lds4(xrow + kb);
            ax = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds4(wxr + kb), bx, ax, 0, 0, 0);
            aa = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds4(war + kb), bx, aa, 0, 0, 0);
        }
        const int tok = wave * 16 + col;
        if (tok < valid) {
            const int o = blk * Db + mt * 16 + 4 * grp;  // four consecutive channels
            const float4 bxv = *reinterpret_cast<const float4*>(b_x + o);
            const float4 bav = *reinterpret_cast<const float4*>(b_a + o);
            const size_t dst = (t0 + tok) * D + o;
            *reinterpret_cast<uint2*>(lx + dst) =
                make_uint2(bf16_pair(ax[0] + bxv.x, ax[1] + bxv.y), bf16_pair(ax[2] + bxv.z, ax[3] + bxv.w));
            *reinterpret_cast<uint2*>(la + dst) =
                make_uint2(bf16_pair(aa[0] + bav.x, aa[1] + bav.y), bf16_pair(aa[2] + bav.z, aa[3] + bav.w));
        }
    }
}

// ------------------------------------------------------------ dx (adjoint)
// dx^T[k][t] = sum_o W^T[k][o] dl^T[o][t] summed over both gates (one gate
// at a time through LDS: W^T rows are inputs k, dl rows are tokens), then
// added to dx_in.  Each wave owns 16 tokens and every input tile.
constexpr int GP_MT_MAX = 10;  // Db <= 160

template <bool F32>
__global__ __launch_bounds__(GP_THREADS) void gate_proj_dx_kernel(
    int BL, int D, const uint16_t* __restrict__ w_x, const uint16_t* __restrict__ w_a,
    const void* __restrict__ dlx, const void* __restrict__ dla, const void* dx_in, void* dx_out) {
    extern __shared__ uint16_t gp_lds[];
    const int Db = D / 16, RS = Db + GP_PAD;
    uint16_t* sW = gp_lds;                                   // W_g^T [k][o] bf16
    float* sDf = reinterpret_cast<float*>(sW + Db * RS);     // F32: dl_g [t][o]
    uint16_t* sDb = sW + Db * RS;                            // BF16: dl_g [t][o]
    const int blk = blockIdx.y;
    const size_t t0 = (size_t)blockIdx.x * GP_TT;
    const int valid = (int)min((size_t)GP_TT, (size_t)BL - t0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int MT = Db / 16;
    const int tok = wave * 16 + col;
    v4f acc[GP_MT_MAX];
#pragma unroll
    for (int m = 0; m < GP_MT_MAX; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < 2; ++g) {
        const uint16_t* w = (g ? w_a : w_x) + (size_t)blk * Db * Db;
        const void* dl = g ? dla : dlx;
        if (g) __syncthreads();  // the first gate's tiles are no longer read
        for (int c = threadIdx.x; c < Db * Db; c += GP_THREADS) {
            const int o = c / Db, k = c - o * Db;
            sW[k * RS + o] = w[c];
        }
        if (F32) {
            const int per_row = Db / 4;
            for (int c = threadIdx.x; c < GP_TT * per_row; c += GP_THREADS) {
                const int r = c / per_row, k4 = (c - r * per_row) * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (r < valid)
                    v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(dl) + (t0 + r) * D +
                                                         (size_t)blk * Db + k4);
                *reinterpret_cast<float4*>(sDf + (size_t)r * RS + k4) = v;
            }
        } else {
            stage_rows(sDb, reinterpret_cast<const uint16_t*>(dl) + t0 * D + (size_t)blk * Db, D, GP_TT, valid, Db);
        }
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < GP_MT_MAX; ++mt) {
            if (mt >= MT) continue;
            v4f a = acc[mt];
            if (F32) {
                // 16x16x4: lane l holds A[l%16][l/16], B[l/16][l%16]
                for (int kb = 0; kb < Db; kb += 4) {
                    const int o = kb + grp;
                    const float av = __uint_as_float((uint32_t)sW[(mt * 16 + col) * RS + o] << 16);
                    a = __builtin_amdgcn_mfma_f32_16x16x4f32(av, sDf[(size_t)tok * RS + o], a, 0, 0, 0);
                }
            } else {
                const uint16_t* wr = sW + (mt * 16 + col) * RS + 4 * grp;
                const uint16_t* dr = sDb + (size_t)tok * RS + 4 * grp;
                for (int kb = 0; kb < Db; kb += 16)
                    a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds4(wr + kb), lds4(dr + kb), a, 0, 0, 0);
            }
            acc[mt] = a;
        }
    }
    if (tok >= valid) return;
#pragma unroll
    for (int mt = 0; mt < GP_MT_MAX; ++mt) {
        if (mt >= MT) continue;
        const size_t dst = (t0 + tok) * D + (size_t)blk * Db + mt * 16 + 4 * grp;
        if (F32) {
            const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(dx_in) + dst);
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(dx_out) + dst) =
                make_float4(a.x + acc[mt][0], a.y + acc[mt][1], a.z + acc[mt][2], a.w + acc[mt][3]);
        } else {
            const uint2 a = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(dx_in) + dst);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dx_out) + dst) =
                make_uint2(bf16_pair(bf16_lo(a.x) + acc[mt][0], bf16_hi(a.x) + acc[mt][1]),
                           bf16_pair(bf16_lo(a.y) + acc[mt][2], bf16_hi(a.y) + acc[mt][3]));
        }
    }
}

// ------------------------------------------------------- dW, db (adjoint)
// Partial sums over one token range r: dW^(r)[o][k] = sum_t dl[t][o] x[t][k].
// grid (n_ranges, 16 blocks, ceil(MT / 4) output-tile groups): wave w owns
// output tile ot = 4 * group + w (16 outputs) against every input tile, for
// both gates.  A = dl^T (rows o), B = x (columns k), both staged transposed
// (rows = channels, columns = tokens) so fragment reads are contiguous.
template <bool F32>
__global__ __launch_bounds__(GP_THREADS) void gate_proj_dw_kernel(
    int BL, int D, int range, const uint16_t* __restrict__ x, const void* __restrict__ dlx,
    const void* __restrict__ dla, float* __restrict__ dw_part, float* __restrict__ db_part) {
    extern __shared__ uint16_t gp_lds[];
    const int Db = D / 16;
    const int TS = GP_TT + GP_PAD;
    uint16_t* sX = gp_lds;                                  // x^T [k][t] bf16, all Db inputs
    float* sLf = reinterpret_cast<float*>(sX + Db * TS);    // F32: dl^T [2][64 outputs][t]
    uint16_t* sLb = sX + Db * TS;                           // BF16: same
    const int r = blockIdx.x, blk = blockIdx.y, og = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int MT = Db / 16;
    const int o0 = og * 64;                                 // first output of the group
    const int ot = 4 * og + wave;                           // this wave's output tile
    const size_t tr0 = (size_t)r * range;
    const size_t tr1 = min((size_t)BL, tr0 + range);
    v4f acc[2][GP_MT_MAX];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int n = 0; n < GP_MT_MAX; ++n) acc[g][n] = v4f{0.f, 0.f, 0.f, 0.f};
    float dbs[2] = {0.f, 0.f};  // thread j < 64: column sums of output o0 + j
    for (size_t t0 = tr0; t0 < tr1; t0 += GP_TT) {
        const int valid = (int)min((size_t)GP_TT, tr1 - t0);
        __syncthreads();
        for (int c = threadIdx.x; c < GP_TT * Db; c += GP_THREADS) {
            const int t = c / Db, k = c - t * Db;
            sX[k * TS + t] = t < valid ? x[(t0 + t) * D + (size_t)blk * Db + k] : (uint16_t)0;
        }
        for (int c = threadIdx.x; c < 2 * GP_TT * 64; c += GP_THREADS) {
            const int g = c / (GP_TT * 64), rem = c - g * GP_TT * 64;
            const int t = rem / 64, j = rem - t * 64;
            const bool ok = t < valid && o0 + j < Db;
            const size_t src = (t0 + t) * D + (size_t)blk * Db + o0 + j;
            const void* dl = g ? dla : dlx;
            if (F32) sLf[((size_t)g * 64 + j) * TS + t] = ok ? reinterpret_cast<const float*>(dl)[src] : 0.f;
            else sLb[(g * 64 + j) * TS + t] = ok ? reinterpret_cast<const uint16_t*>(dl)[src] : (uint16_t)0;
        }
        __syncthreads();
        if (threadIdx.x < 64) {
            const int j = threadIdx.x;
            for (int t = 0; t < valid; ++t) {
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    dbs[g] += F32 ? sLf[((size_t)g * 64 + j) * TS + t]
                                  : __uint_as_float((uint32_t)sLb[(g * 64 + j) * TS + t] << 16);
            }
        }
        if (ot < MT) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int n = 0; n < GP_MT_MAX; ++n) {
                    if (n >= MT) continue;
                    v4f a = acc[g][n];
                    if (F32) {
                        for (int kt = 0; kt < GP_TT; kt += 4) {
                            const float av = sLf[((size_t)g * 64 + wave * 16 + col) * TS + kt + grp];
                            const float bv = __uint_as_float((uint32_t)sX[(n * 16 + col) * TS + kt + grp] << 16);
                            a = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, a, 0, 0, 0);
                        }
                    } else {
                        const uint16_t* ar = sLb + (g * 64 + wave * 16 + col) * TS + 4 * grp;
                        const uint16_t* br = sX + (n * 16 + col) * TS + 4 * grp;
                        for (int kt = 0; kt < GP_TT; kt += 16)
                            a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds4(ar + kt), lds4(br + kt), a, 0, 0, 0);
                    }
                    acc[g][n] = a;
                }
        }
    }
    // D[o][k]: lane holds o = 16 ot + 4 grp + i, k = 16 n + col
    if (ot < MT) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int n = 0; n < GP_MT_MAX; ++n) {
                if (n >= MT) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t o = (size_t)ot * 16 + 4 * grp + i;
                    dw_part[((((size_t)r * 2 + g) * 16 + blk) * Db + o) * Db + n * 16 + col] = acc[g][n][i];
                }
            }
    }
    if (threadIdx.x < 64 && o0 + (int)threadIdx.x < Db) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
            db_part[((size_t)r * 2 + g) * D + (size_t)blk * Db + o0 + threadIdx.x] = dbs[g];
    }
}

// Sum of the range partials in range order (FP64): dw [2][16][Db][Db], db [2][D].
__global__ __launch_bounds__(256) void gate_proj_reduce_kernel(int n_ranges, int nw, int D,
                                                               const float* __restrict__ dw_part,
                                                               const float* __restrict__ db_part,
                                                               float* __restrict__ dw_x, float* __restrict__ dw_a,
                                                               float* __restrict__ db_x, float* __restrict__ db_a) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int half = nw / 2;
    if (e < nw) {
        double s = 0.0;
        for (int r = 0; r < n_ranges; ++r) s += dw_part[(size_t)r * nw + e];
        if (e < half) dw_x[e] = (float)s;
        else dw_a[e - half] = (float)s;
    } else if (e < nw + 2 * D) {
        const int f = e - nw;
        double s = 0.0;
        for (int r = 0; r < n_ranges; ++r) s += db_part[(size_t)r * 2 * D + f];
        if (f < D) db_x[f] = (float)s;
        else db_a[f - D] = (float)s;
    }
}

}  // namespace

int gate_proj_ranges(int BL) { return (int)std::max<int64_t>(1, ceil_div(BL, GP_RANGE)); }

size_t gate_proj_fwd_lds(int D) {
    const int Db = D / 16;
    return (size_t)(2 * Db + GP_TT) * (Db + GP_PAD) * 2;
}

hipError_t launch_gate_proj_fwd(int BL, int D, const void* x, const void* w_x, const float* b_x,
                                const void* w_a, const float* b_a, void* lx, void* la, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(BL, GP_TT), 16);
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gate_proj_fwd_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)gate_proj_fwd_lds(D));
    if (e != hipSuccess) return e;
    LRS_LAUNCH(K_GATE_PROJ, gate_proj_fwd_kernel, grid, dim3(GP_THREADS), gate_proj_fwd_lds(D), s, BL, D,
               (const uint16_t*)x, (const uint16_t*)w_x, b_x, (const uint16_t*)w_a, b_a, (uint16_t*)lx,
               (uint16_t*)la);
    return hipGetLastError();
}

size_t gate_proj_dx_lds(int D, int f32) {
    const int Db = D / 16;
    return (size_t)Db * (Db + GP_PAD) * 2 + (size_t)GP_TT * (Db + GP_PAD) * (f32 ? 4 : 2);
}

size_t gate_proj_dw_lds(int D, int f32) {
    const int Db = D / 16;
    return (size_t)Db * (GP_TT + GP_PAD) * 2 + (size_t)2 * 64 * (GP_TT + GP_PAD) * (f32 ? 4 : 2);
}

template <class F>
static hipError_t allow_lds(F* kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

hipError_t launch_gate_proj_bwd(int BL, int D, const void* x, const void* w_x, const void* w_a, const void* dlx,
                                const void* dla, int f32, const void* dx_in, void* dx_out, float* dw_x,
                                float* db_x, float* dw_a, float* db_a, float* dw_part, float* db_part,
                                hipStream_t s) {
    const int Db = D / 16;
    const size_t lds_dx = gate_proj_dx_lds(D, f32), lds_dw = gate_proj_dw_lds(D, f32);
    const int nr = gate_proj_ranges(BL);
    const dim3 gdx((unsigned)ceil_div(BL, GP_TT), 16), gdw((unsigned)nr, 16, (unsigned)ceil_div(Db / 16, 4));
    hipError_t e;
    if (f32) {
        if ((e = allow_lds(gate_proj_dx_kernel<true>, lds_dx)) != hipSuccess) return e;
        if ((e = allow_lds(gate_proj_dw_kernel<true>, lds_dw)) != hipSuccess) return e;
        LRS_LAUNCH(K_GATE_PROJ_BWD, gate_proj_dx_kernel<true>, gdx, dim3(GP_THREADS), lds_dx, s, BL, D,
                   (const uint16_t*)w_x, (const uint16_t*)w_a, dlx, dla, dx_in, dx_out);
        LRS_LAUNCH(K_GATE_PROJ_BWD, gate_proj_dw_kernel<true>, gdw, dim3(GP_THREADS), lds_dw, s, BL, D, GP_RANGE,
                   (const uint16_t*)x, dlx, dla, dw_part, db_part);
    } else {
        if ((e = allow_lds(gate_proj_dx_kernel<false>, lds_dx)) != hipSuccess) return e;
        if ((e = allow_lds(gate_proj_dw_kernel<false>, lds_dw)) != hipSuccess) return e;
        LRS_LAUNCH(K_GATE_PROJ_BWD, gate_proj_dx_kernel<false>, gdx, dim3(GP_THREADS), lds_dx, s, BL, D,
                   (const uint16_t*)w_x, (const uint16_t*)w_a, dlx, dla, dx_in, dx_out);
        LRS_LAUNCH(K_GATE_PROJ_BWD, gate_proj_dw_kernel<false>, gdw, dim3(GP_THREADS), lds_dw, s, BL, D,
                   GP_RANGE, (const uint16_t*)x, dlx, dla, dw_part, db_part);
    }
    const int nw = 2 * 16 * Db * Db;
    LRS_LAUNCH(K_GATE_PROJ_BWD, gate_proj_reduce_kernel, dim3((unsigned)ceil_div(nw + 2 * D, 256)), dim3(256), 0,
               s, nr, nw, D, dw_part, db_part, dw_x, dw_a, db_x, db_a);
    return hipGetLastError();
}

}  // namespace lrs
