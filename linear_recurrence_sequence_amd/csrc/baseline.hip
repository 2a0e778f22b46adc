// baseline.hip -- the two comparison scans of the scan-latency experiment,
// forward only, for the SAMU and RG-LRU recurrences on MI355X.
//
// Page 'Griffin 第 4、5 节 H800 对照协议', experiment-coverage matrix, the
// Fig. 8(a) row: at B=8, width 1024, L=2K..16K the exact chunked scan is
// timed against a per-channel on-chip sequential scan and associative
// (log-depth) scans, for SAMU and for RG-LRU.  Both baselines here compute
// the same recurrences as the chunked library path (page 'SAMU 与 RG-LRU 的
// H800 训练性能对比', sections 04 and 05):
//   * sequential: one lane per (batch row, mode or channel) walks all L
//     tokens in order, its state in a register; the drive words of the next
//     SEQ_TB tokens are requested before they are needed;
//   * associative: the recursive pairwise scan over HBM.  With e_t the token
//     maps h -> A_t h + B_t (A_t = lambda_t or a_t) and (f o g) = f after g,
//       level k+1 element j = e_{2j+1} o e_{2j}          (reduce, k = 0..),
//     the inclusive prefixes P at level k follow from those P' of level k+1:
//       P_{2j+1} = P'_j,  P_{2j} = e_{2j} o P'_{j-1},  P_0 = e_0  (expand),
//     log2(L) reduce and log2(L) expand launches in all.  Level 0 is never
//     stored: its reduce forms e_t from the inputs and its expand writes
//     y_t = P_t(h0) directly.
// Lanes run over modes (SAMU) or channels (RG-LRU) so every access to a
// [B, L, *] row is contiguous across the wave.
#include "common.hpp"

namespace lrs {
namespace {

constexpr int BL_THREADS = 256;
constexpr int SEQ_THREADS = 64;
constexpr int SEQ_TB = 16;  // tokens whose drive words are requested together
constexpr float LOG2E_F = 1.4426950408889634f;

// ------------------------------------------------------------ elements ---
struct CAff {  // complex affine map h -> a h + b
    cf a, b;
    __device__ CAff after(const CAff& f) const { return {cmul(a, f.a), cfma(a, f.b, b)}; }
    __device__ cf apply(cf h) const { return cfma(a, h, b); }
    __device__ static CAff load(const float4* p, size_t i) {
        const float4 v = p[i];
        return {{v.x, v.y}, {v.z, v.w}};
    }
    __device__ void store(float4* p, size_t i) const { p[i] = make_float4(a.re, a.im, b.re, b.im); }
};

struct RAff {  // real affine map h -> a h + b
    float a, b;
    __device__ RAff after(const RAff& f) const { return {a * f.a, fmaf(a, f.b, b)}; }
    __device__ float apply(float h) const { return fmaf(a, h, b); }
    __device__ static RAff load(const float2* p, size_t i) {
        const float2 v = p[i];
        return {v.x, v.y};
    }
    __device__ void store(float2* p, size_t i) const { p[i] = make_float2(a, b); }
};

// token maps of the two recurrences
struct SamuTok {
    const TokenCtl* ctl;      // [B, L]
    const uint32_t* drive;    // [B, L, M] complex BF16 words
    const float4* mtab;
    int L, W;                 // W = M
    __device__ CAff operator()(int b, int t, int m, const ModeConst& k) const {
        const TokenCtl c = ctl[(size_t)b * L + t];
        const uint32_t w = drive[((size_t)b * L + t) * W + m];
        return {mode_lambda(k, c.E, c.C, c.S), {bf16_lo(w), bf16_hi(w)}};
    }
};

struct RgConst {
    float k8;  // -8 softplus(alpha) log2(e)
};

__device__ __forceinline__ RgConst rg_const(float alpha) {
    const float sp = alpha > 20.f ? alpha + log1pf(expf(-alpha)) : log1pf(expf(alpha));
    return {-8.0f * sp * LOG2E_F};
}

__device__ __forceinline__ float bf16_at(const uint16_t* p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}

struct RgTok {
    const uint16_t *x, *lx, *la;  // [B, L, D] BF16
    const unsigned char* reset;   // [B, L] or NULL
    int L, W;                     // W = D
    __device__ RAff operator()(int b, int t, int d, const RgConst& k) const {
        const size_t i = ((size_t)b * L + t) * W + d;
        const float gx = 1.0f / (1.0f + expf(-bf16_at(lx, i)));
        const float ga = 1.0f / (1.0f + expf(-bf16_at(la, i)));
        const float a = exp2f(k.k8 * ga);
        const bool rs = reset && reset[(size_t)b * L + t];
        const float m = rs ? 1.0f : sqrtf(fmaxf(1.0f - a * a, 0.0f));
        return {rs ? 0.0f : a, bf16_at(x, i) * gx * m};
    }
};

// ------------------------------------------------------ sequential scans ---
__global__ __launch_bounds__(SEQ_THREADS) void samu_seq_scan_kernel(
    int L, int M, const TokenCtl* __restrict__ ctl, const uint32_t* __restrict__ drive,
    const float4* __restrict__ mtab, const float2* __restrict__ z0, void* __restrict__ y, int y_f32,
    float2* __restrict__ z_final) {
    const int m = blockIdx.x * SEQ_THREADS + threadIdx.x;
    const int b = blockIdx.y;
    if (m >= M) return;
    const ModeConst k = load_mode(mtab, m);
    cf z = z0 ? cf{z0[(size_t)b * M + m].x, z0[(size_t)b * M + m].y} : cf{0.f, 0.f};
    const size_t row0 = (size_t)b * L;
    for (int t0 = 0; t0 < L; t0 += SEQ_TB) {
        const int n = min(SEQ_TB, L - t0);
        uint32_t w[SEQ_TB];
#pragma unroll
        for (int i = 0; i < SEQ_TB; ++i) w[i] = i < n ? drive[(row0 + t0 + i) * M + m] : 0u;
#pragma unroll
        for (int i = 0; i < SEQ_TB; ++i) {
            if (i < n) {
                const TokenCtl c = ctl[row0 + t0 + i];
                z = cfma(mode_lambda(k, c.E, c.C, c.S), z, {bf16_lo(w[i]), bf16_hi(w[i])});
                const size_t o = (row0 + t0 + i) * M + m;
                if (y_f32) reinterpret_cast<float2*>(y)[o] = make_float2(z.re, z.im);
                else reinterpret_cast<uint32_t*>(y)[o] = pack_bf16x2(z.re, z.im);
            }
        }
    }
    if (z_final) z_final[(size_t)b * M + m] = make_float2(z.re, z.im);
}

__global__ __launch_bounds__(SEQ_THREADS) void rglru_seq_scan_kernel(
    RgTok tk, const float* __restrict__ alpha, const float* __restrict__ h0, void* __restrict__ y, int y_f32,
    float* __restrict__ h_final) {
    const int d = blockIdx.x * SEQ_THREADS + threadIdx.x;
    const int b = blockIdx.y;
    const int D = tk.W;
    if (d >= D) return;
    const RgConst k = rg_const(alpha[d]);
    float h = h0 ? h0[(size_t)b * D + d] : 0.f;
    for (int t0 = 0; t0 < tk.L; t0 += SEQ_TB) {
        const int n = min(SEQ_TB, tk.L - t0);
        uint16_t xs[SEQ_TB], lxs[SEQ_TB], las[SEQ_TB];
#pragma unroll
        for (int i = 0; i < SEQ_TB; ++i) {
            const size_t o = ((size_t)b * tk.L + t0 + min(i, n - 1)) * D + d;
            xs[i] = tk.x[o];
            lxs[i] = tk.lx[o];
            las[i] = tk.la[o];
        }
#pragma unroll
        for (int i = 0; i < SEQ_TB; ++i) {
            if (i < n) {
                const float gx = 1.0f / (1.0f + expf(-__uint_as_float((uint32_t)lxs[i] << 16)));
                const float ga = 1.0f / (1.0f + expf(-__uint_as_float((uint32_t)las[i] << 16)));
                const float a = exp2f(k.k8 * ga);
                const bool rs = tk.reset && tk.reset[(size_t)b * tk.L + t0 + i];
                const float m = rs ? 1.0f : sqrtf(fmaxf(1.0f - a * a, 0.0f));
                h = fmaf(rs ? 0.0f : a, h, __uint_as_float((uint32_t)xs[i] << 16) * gx * m);
                const size_t o = ((size_t)b * tk.L + t0 + i) * D + d;
                if (y_f32) reinterpret_cast<float*>(y)[o] = h;
                else reinterpret_cast<__bf16*>(y)[o] = (__bf16)h;
            }
        }
    }
    if (h_final) h_final[(size_t)b * D + d] = h;
}

// ----------------------------------------------------- associative scans ---
// Level arrays of n_k maps each, [B, n_k, W]; level 0 is the tokens.
// reduce: out[j] = in[2j+1] o in[2j], j < n_k / 2.
template <class Aff, class Vec, class Tok, class Const, Const (*MK)(const float*, int)>
__global__ __launch_bounds__(BL_THREADS) void assoc_reduce_kernel(int n_in, int n_out, int W, int gw, Tok tk,
                                                                  const float* __restrict__ kp,
                                                                  const Vec* __restrict__ in,
                                                                  Vec* __restrict__ out) {
    // grid x = (element blocks) x (pairs), so the pair count is not bound by grid y
    const int j = blockIdx.x / gw;
    const int w = (blockIdx.x - j * gw) * BL_THREADS + threadIdx.x;
    const int b = blockIdx.y;
    if (w >= W) return;
    Aff e0, e1;
    if (in == nullptr) {  // level 0: the token maps themselves
        const Const k = MK(kp, w);
        e0 = tk(b, 2 * j, w, k);
        e1 = tk(b, 2 * j + 1, w, k);
    } else {
        e0 = Aff::load(in, ((size_t)b * n_in + 2 * j) * W + w);
        e1 = Aff::load(in, ((size_t)b * n_in + 2 * j + 1) * W + w);
    }
    e1.after(e0).store(out, ((size_t)b * n_out + j) * W + w);
}

// expand: given inclusive prefixes P' of level k+1 (in `up`, n_up = n_k / 2
// maps), turn level k into its inclusive prefixes in place; at level 0
// (lvl == nullptr) write y_t = P_t(h0) and the final state instead.
template <class Aff, class Vec, class St, class Tok, class Const, Const (*MK)(const float*, int),
          class Out>
__global__ __launch_bounds__(BL_THREADS) void assoc_expand_kernel(int n, int n_up, int W, int gw, Tok tk,
                                                                  const float* __restrict__ kp,
                                                                  Vec* __restrict__ lvl,
                                                                  const Vec* __restrict__ up, Out out) {
    const int j = blockIdx.x / gw;  // pair j covers elements 2j, 2j+1
    const int w = (blockIdx.x - j * gw) * BL_THREADS + threadIdx.x;
    const int b = blockIdx.y;
    if (w >= W || 2 * j >= n) return;
    // P_{2j} = e_{2j} o P'_{j-1} (e_0 alone for j = 0); P_{2j+1} = P'_j
    Aff e;
    if (lvl == nullptr) e = tk(b, 2 * j, w, MK(kp, w));
    else e = Aff::load(lvl, ((size_t)b * n + 2 * j) * W + w);
    const Aff pe = j > 0 ? e.after(Aff::load(up, ((size_t)b * n_up + j - 1) * W + w)) : e;
    const bool has_odd = 2 * j + 1 < n;
    Aff po;
    if (has_odd) po = Aff::load(up, ((size_t)b * n_up + j) * W + w);
    if (lvl != nullptr) {
        pe.store(lvl, ((size_t)b * n + 2 * j) * W + w);
        if (has_odd) po.store(lvl, ((size_t)b * n + 2 * j + 1) * W + w);
    } else {
        out.put(b, 2 * j, w, pe);
        if (has_odd) out.put(b, 2 * j + 1, w, po);
    }
}

__device__ ModeConst samu_mk(const float* mtab, int m) { return load_mode(reinterpret_cast<const float4*>(mtab), m); }
__device__ RgConst rg_mk(const float* alpha, int d) { return rg_const(alpha[d]); }

struct SamuOut {
    const float2* z0;
    void* y;
    float2* z_final;
    int L, M, f32;
    __device__ void put(int b, int t, int m, const CAff& P) const {
        const cf h0 = z0 ? cf{z0[(size_t)b * M + m].x, z0[(size_t)b * M + m].y} : cf{0.f, 0.f};
        const cf z = P.apply(h0);
        const size_t o = ((size_t)b * L + t) * M + m;
        if (f32) reinterpret_cast<float2*>(y)[o] = make_float2(z.re, z.im);
        else reinterpret_cast<uint32_t*>(y)[o] = pack_bf16x2(z.re, z.im);
        if (z_final && t == L - 1) z_final[(size_t)b * M + m] = make_float2(z.re, z.im);
    }
};

struct RgOut {
    const float* h0;
    void* y;
    float* h_final;
    int L, D, f32;
    __device__ void put(int b, int t, int d, const RAff& P) const {
        const float h = P.apply(h0 ? h0[(size_t)b * D + d] : 0.f);
        const size_t o = ((size_t)b * L + t) * D + d;
        if (f32) reinterpret_cast<float*>(y)[o] = h;
        else reinterpret_cast<__bf16*>(y)[o] = (__bf16)h;
        if (h_final && t == L - 1) h_final[(size_t)b * D + d] = h;
    }
};

// Level sizes n_0 = L, n_{k+1} = n_k / 2 down to 1, and their offsets (in
// maps of one batch row and element) in the level workspace.
int assoc_levels(int L, int* n, size_t* off) {
    int k = 0;
    size_t o = 0;
    n[0] = L;
    off[0] = 0;
    while (n[k] > 1) {
        n[k + 1] = n[k] / 2;
        off[k + 1] = o;
        o += (size_t)n[k + 1];
        ++k;
    }
    return k;  // number of reduce levels; n[k] == 1
}

template <class Aff, class Vec, class St, class Tok, class Const, Const (*MK)(const float*, int), class Out>
hipError_t run_assoc(int B, int L, int W, Tok tk, const float* kp, Vec* levels, Out out, hipStream_t s) {
    int n[40];
    size_t off[40];
    const int top = assoc_levels(L, n, off);
    auto lv = [&](int k) -> Vec* { return k == 0 ? nullptr : levels + off[k] * (size_t)B * W; };
    const int gw = (int)ceil_div(W, BL_THREADS);
    for (int k = 0; k < top; ++k)
        LRS_LAUNCH(K_BASE_ASSOC, (assoc_reduce_kernel<Aff, Vec, Tok, Const, MK>),
                   dim3((unsigned)((int64_t)gw * n[k + 1]), B), dim3(BL_THREADS), 0, s, n[k], n[k + 1], W, gw,
                   tk, kp, (const Vec*)lv(k), lv(k + 1));
    if (top == 0) {
        // a single token: its map is its own prefix; expand with no upper level
        LRS_LAUNCH(K_BASE_ASSOC, (assoc_expand_kernel<Aff, Vec, St, Tok, Const, MK, Out>), dim3(gw, B),
                   dim3(BL_THREADS), 0, s, 1, 0, W, gw, tk, kp, (Vec*)nullptr, (const Vec*)nullptr, out);
        return hipGetLastError();
    }
    for (int k = top - 1; k >= 0; --k)
        LRS_LAUNCH(K_BASE_ASSOC, (assoc_expand_kernel<Aff, Vec, St, Tok, Const, MK, Out>),
                   dim3((unsigned)((int64_t)gw * ceil_div(n[k], 2)), B), dim3(BL_THREADS), 0, s, n[k], n[k + 1],
                   W, gw, tk, kp, lv(k), (const Vec*)lv(k + 1), out);
    return hipGetLastError();
}

}  // namespace

size_t assoc_level_maps(int L) {
    int n[40];
    size_t off[40];
    const int top = assoc_levels(L, n, off);
    return top == 0 ? 0 : off[top] + (size_t)n[top];
}

hipError_t launch_samu_baseline(int variant, const SamuParams& p, const float* ctl, const float* mtab,
                                float* levels, void* y, int y_f32, float* z_final, hipStream_t s) {
    if (variant == 0) {
        LRS_LAUNCH(K_BASE_SEQ, samu_seq_scan_kernel, dim3((unsigned)ceil_div(p.M, SEQ_THREADS), p.B),
                   dim3(SEQ_THREADS), 0, s, p.L, p.M, (const TokenCtl*)ctl, (const uint32_t*)p.b,
                   (const float4*)mtab, (const float2*)p.z0, y, y_f32, (float2*)z_final);
        return hipGetLastError();
    }
    const SamuTok tk{(const TokenCtl*)ctl, (const uint32_t*)p.b, (const float4*)mtab, p.L, p.M};
    const SamuOut out{(const float2*)p.z0, y, (float2*)z_final, p.L, p.M, y_f32};
    return run_assoc<CAff, float4, cf, SamuTok, ModeConst, samu_mk, SamuOut>(p.B, p.L, p.M, tk, mtab,
                                                                              (float4*)levels, out, s);
}

hipError_t launch_rglru_baseline(int variant, const RglruParams& p, float* levels, void* y, int y_f32,
                                 float* h_final, hipStream_t s) {
    const RgTok tk{(const uint16_t*)p.x, (const uint16_t*)p.lx, (const uint16_t*)p.la, p.reset, p.L, p.D};
    if (variant == 0) {
        LRS_LAUNCH(K_BASE_SEQ, rglru_seq_scan_kernel, dim3((unsigned)ceil_div(p.D, SEQ_THREADS), p.B),
                   dim3(SEQ_THREADS), 0, s, tk, p.alpha, p.h0, y, y_f32, h_final);
        return hipGetLastError();
    }
    const RgOut out{p.h0, y, h_final, p.L, p.D, y_f32};
    return run_assoc<RAff, float2, float, RgTok, RgConst, rg_mk, RgOut>(p.B, p.L, p.D, tk, p.alpha,
                                                                        (float2*)levels, out, s);
}

}  // namespace lrs
