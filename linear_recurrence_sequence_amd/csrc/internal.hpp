// internal.hpp -- host-side plumbing shared by the kernel files and the C ABI:
// launch geometry, the optional per-kernel event profiler, and the launcher
// declarations of every kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lrs {

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ profiler ---
// When enabled, every kernel launch is bracketed by a pair of HIP events on
// the launch stream; scan_profile_* in the C ABI read the sums back.
enum KernelId {
    K_SAMU_CONTROLLER = 0,
    K_SAMU_SUMMARY,
    K_PREFIX_GROUPS,
    K_PREFIX_OUTER,
    K_PREFIX_ENTRIES,
    K_SAMU_REPLAY,
    K_SAMU_REV_SUMMARY,
    K_SAMU_BWD_REPLAY,
    K_SAMU_CTL_BWD,
    K_SAMU_PARAMS,
    K_RGLRU_SUMMARY,
    K_RGLRU_REPLAY,
    K_RGLRU_REV_SUMMARY,
    K_RGLRU_BWD_REPLAY,
    K_RGLRU_ALPHA,
    K_SAMU_DECODE,
    K_BASE_SEQ,
    K_BASE_ASSOC,
    K_GATE_PROJ,
    K_GATE_PROJ_DX,
    K_GATE_PROJ_DW,
    K_GATE_PROJ_REDUCE,
    K_SAMU_FWD_SCAN,
    K_SAMU_BWD_SCAN,
    K_CLEAR,
    K_GATE_PROJ_ADJ,
    K_RGLRU_FWD_SCAN,
    K_RGLRU_BWD_SCAN,
    K_NUM_KERNELS
};

const char* kernel_name(int id);
// sets the thread-local text scan_last_error() returns; returns st
int set_last_error(int st, const char* msg);
bool profiler_enabled();
void profiler_before(int id, hipStream_t s);
void profiler_after(int id, hipStream_t s);

#define LRS_LAUNCH(ID, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                        \
    do {                                                                                 \
        const bool _prof = ::lrs::profiler_enabled();                                    \
        if (_prof) ::lrs::profiler_before((ID), (STREAM));                               \
        hipLaunchKernelGGL(KERNEL, (GRID), (BLOCK), (SHMEM), (STREAM), __VA_ARGS__);     \
        if (_prof) ::lrs::profiler_after((ID), (STREAM));                                \
    } while (0)

// ------------------------------------------------------------- layouts ---
// Chunking of one scan: C chunks of K tokens (last one K_c = L - (C-1)K),
// grouped G chunks at a time into NG groups for the two-level prefix.
struct Chunking {
    int B, L, K, C, G, NG;
};

// --------------------------------------------------- prefix (all scans) ---
// Element type of a scan: 1 = real (RG-LRU channels), 2 = complex (SAMU modes).
// Chunk summaries in chunk order:
//   real:    full = [B, C, W] (A, B) pairs;
//   complex: bpart = [B, C, W] complex B parts, chunk = [B, C] float4
//            (G_c, cos D_c, sin D_c, 0), mtab = the mode table (the chunk
//            phasors e^{i K theta}, e^{i K_last theta} and kappa per mode).
struct PrefixSummaries {
    const float* full;
    const float* bpart;
    const float* chunk;
    const float* mtab;
};
// gsum:    workspace of 3*ELEM floats per (batch, group, element): [B, NG, W]
//          group summaries U_g in processing order, then [B, NG, W] states
//          entering each group (unused with a single group)
// init:    [B, W] initial state (NULL = 0)
// entries: [B, C, W] state entering each chunk (ELEM floats each); for an
//          adjoint scan (reverse) the cotangent arriving after its last token
hipError_t launch_prefix(int elem, bool reverse, const Chunking& ch, int W, const PrefixSummaries& sm,
                         float* gsum, const float* init, float* entries, hipStream_t s);

// ---------------------------------------------------------------- SAMU ---
struct SamuParams {
    int B, L, D, M;
    const void* x_sel;       // bf16 [B, L, D]
    const void* b;           // bf16 [B, L, M, 2]
    const float* w_phi;      // [D+1]
    const float* w_r;        // [D+1]
    const float* a_phi;      // [1]
    const float* a_r;        // [1]
    const float* nu;         // [M]
    const float* theta;      // [M]
    const float* z0;         // [B, M, 2] or NULL
};

// saved forward record (per token): p, r, u = (x~ . w^_phi, x~ . w^_r),
// ctl = (E, C, S, d); per mode: the four-float4 constant table mtab;
// inv_norm (NULL: not written): floats 0-1 = (1/||w_phi||, 1/||w_r||), floats
// 4-7 = the FP64 squared norms (||w_phi||^2, ||w_r||^2) summed in a fixed order.
// crec (NULL: not written): [B, C] float4 record of every chunk, (G_c, cos D_c,
// sin D_c, 0) with G_c = sum E_t and D_c = sum d_t in token order
// crec: per-chunk records (NULL: not written); clear: clear_bytes (a multiple
// of 16) zeroed after the controller's own work (NULL: none)
hipError_t launch_samu_controller(const SamuParams& p, const Chunking& ch, float* p_out, float* r_out,
                                  float* u_out, float* ctl, float* mtab, float* inv_norm, float* crec,
                                  void* clear, size_t clear_bytes, hipStream_t s);
// The backward replay handles a chunk as K / SAMU_BWD_SUB sub-chunks; the
// forward replay keeps the state entering each sub-chunk after the first
// (mid [B, C, samu_mid_states(K), M] complex), so the backward need not run
// the forward recurrence to reach them.
constexpr int SAMU_BWD_SUB = 16;
__host__ __device__ constexpr inline int samu_mid_states(int K) { return K > SAMU_BWD_SUB ? K / SAMU_BWD_SUB - 1 : 0; }

// compressed chunk summaries (forward, or the conjugate reverse summary of
// dy): B parts [B, C, M] complex and per-chunk records [B, C] float4
hipError_t launch_samu_summary(const SamuParams& p, const Chunking& ch, const float* ctl,
                               const float* mtab, const void* drive, bool reverse, float* summ,
                               float* chunk_rec, hipStream_t s);
// replay from the chunk entry states; writes y, z_final and the mid states
hipError_t launch_samu_replay(const SamuParams& p, const Chunking& ch, const float* ctl,
                              const float* mtab, const float* entries, float* mid, void* y, int y_f32,
                              float* z_final, hipStream_t s);
// Grouped path (single-pass scans): a workgroup owns one group of
// ch.G <= SAMU_GROUP_MAX consecutive chunks (processing order) and 64 modes,
// one wave per chunk; groups hand states to each other through
// samu_gscan_pub_bytes() of tagged words that must be zero at launch.
//   gscan:    the whole forward after the controller in one launch (chunk
//             summaries, the state entering the group from the groups before
//             it, the replay, which also writes the entry states [B, C, M]
//             the backward reads); its words are cleared by the controller
//             launch before it (the controller's `clear` argument);
constexpr int SAMU_GROUP_MAX = 16;
// Polls a single-pass scan's wait for another workgroup's hand-off words
// makes before it gives up (the words then read as NaN, so an expired wait
// shows in the outputs instead of passing as a wrong value).  The default
// is far above what a wait takes when the producer runs; the setter exists
// so that tests can force the expiry path.
constexpr int HANDOFF_POLLS_DEFAULT = 1 << 14;
int handoff_poll_limit();
size_t samu_gscan_pub_bytes(const Chunking& ch, int M);
hipError_t launch_samu_gscan(const SamuParams& p, const Chunking& ch, const float* ctl, const float* mtab,
                             const float* chunk_rec, void* pub, float* entries, float* mid, void* y, int y_f32,
                             float* z_final, hipStream_t s);
//   gbscan:   the whole adjoint scan in one launch (reverse summaries, the
//             carry entering each group from the groups after it in time, the
//             backward replay); it clears its words with a small launch of
//             its own first.  mode_part: [B, NG, M] per-group (d nu, d theta)
hipError_t launch_samu_gbscan(const SamuParams& p, const Chunking& ch, const float* ctl, const float* mtab,
                              const float* entries, const float* mid, const float* chunk_rec, const float* dz_final,
                              void* pub, size_t pub_bytes, const void* dy, void* db, int db_f32, float* dz0,
                              float* tok_part, int n_tiles, float* mode_part, hipStream_t s);
// carry_in: [B, C, M] cotangent arriving after each chunk's last token;
// mode_part: [B, C, M] per-chunk (d nu, d theta) partials (gbwd_replay:
// [B, NG, M] per-group sums)
hipError_t launch_samu_bwd_replay(const SamuParams& p, const Chunking& ch, const float* ctl,
                                  const float* mtab, const float* entries, const float* mid,
                                  const float* carry_in, const void* dy, void* db, int db_f32, float* dz0,
                                  float* tok_part, int n_tiles, float* mode_part, hipStream_t s);
int samu_bwd_tiles(int M);
int samu_ctl_tok_per_blk();
int samu_param_columns(int D);
hipError_t launch_samu_ctl_bwd(const SamuParams& p, const float* p_sv, const float* r_sv,
                               const float* u_sv, const float* inv_norm, const float* tok_part, int n_tiles,
                               void* dx_sel, int dx_f32, float* g_part, hipStream_t s);
// g_part: [n_blk, D+4] token-block partials; mode_part: [mode_rows, M] partials
// per chunk (B*C rows) or per group of chunks (B*NG rows, the grouped path)
// wnorm2: the two FP64 squared direction norms the forward controller kept
hipError_t launch_samu_params(const SamuParams& p, const Chunking& ch, const double* wnorm2, const float* g_part,
                              int n_blk, const float* mode_part, int mode_rows, float* dw_phi, float* dw_r,
                              float* da_phi, float* da_r, float* dnu, float* dtheta, hipStream_t s);

// one generation step: z_out = lambda(x_sel) z_in + b, y = z_out (z_in NULL = 0;
// z_out may be z_in); table (NULL: formed per step) from launch_samu_decode_prepare
size_t samu_decode_table_floats(int M);
hipError_t launch_samu_decode_prepare(int D, const float* w_phi, const float* w_r, const float* a_phi,
                                      const float* a_r, const float* nu, const float* theta, float* table,
                                      hipStream_t s);
hipError_t launch_samu_decode(int B, int D, const void* x_sel, const void* b, const float* w_phi,
                              const float* w_r, const float* a_phi, const float* a_r, const float* nu,
                              const float* theta, const float* table, const float* z_in, float* z_out, void* y,
                              int y_f32, hipStream_t s);

// -------------------------------------------------------------- RG-LRU ---
struct RglruParams {
    int B, L, D;
    const void* x;                 // bf16 [B, L, D]
    const void* lx;                // bf16 [B, L, D]
    const void* la;                // bf16 [B, L, D]
    const float* alpha;            // [D]
    const unsigned char* reset;    // [B, L] or NULL
    const float* h0;               // [B, D] or NULL
};

hipError_t launch_rglru_summary(const RglruParams& p, const Chunking& ch, float* summ,
                                hipStream_t s);
hipError_t launch_rglru_replay(const RglruParams& p, const Chunking& ch, const float* entries,
                               void* y, int y_f32, float* h_final, hipStream_t s);
hipError_t launch_rglru_rev_summary(const RglruParams& p, const Chunking& ch, const void* dy,
                                    float* summ, hipStream_t s);
hipError_t launch_rglru_bwd_replay(const RglruParams& p, const Chunking& ch,
                                   const float* entries, const float* carry_in, const void* dy,
                                   void* dx, void* dlx, void* dla, int g_f32, float* dh0,
                                   float* alpha_part, hipStream_t s);
// alpha_part: [rows, D] partials (B*C per-chunk rows, or B*NG per-group rows
// on the single-pass path)
hipError_t launch_rglru_alpha_reduce(const RglruParams& p, int rows, const float* alpha_part, float* dalpha,
                                     hipStream_t s);
// Single-pass grouped scans (K = 16, ch.G <= RG_GROUP_MAX): one workgroup per
// group of consecutive chunks and 64 channel pairs, one wave per chunk; the
// groups hand states to each other through rglru_pub_bytes() of tagged
// words, cleared by the launcher first.
//   gscan:  the whole forward (summaries, hand-off, replay; writes the entry
//           states [B, C, D] the backward reads);
//   gbscan: the whole adjoint scan (reverse summaries, hand-off, backward
//           replay); alpha_part: [B, NG, D] per-group partial sums.
constexpr int RG_GROUP_MAX = 16;
bool rglru_fused(const Chunking& ch);
size_t rglru_pub_bytes(const Chunking& ch, int D);
hipError_t launch_rglru_gscan(const RglruParams& p, const Chunking& ch, void* pub, size_t pub_bytes,
                              float* entries, void* y, int y_f32, float* h_final, hipStream_t s);
hipError_t launch_rglru_gbscan(const RglruParams& p, const Chunking& ch, const float* entries,
                               const float* dh_final, void* pub, size_t pub_bytes, const void* dy, void* dx,
                               void* dlx, void* dla, int g_f32, float* dh0, float* alpha_part, hipStream_t s);
// zeroes `bytes` (a multiple of 16) at p: hand-off words before a single-pass scan
hipError_t launch_clear_words(void* p, size_t bytes, hipStream_t s);

// ------------------------------------------------------ comparison scans ---
// variant 0: per-channel sequential scan; 1: associative (recursive pairwise)
// scan over `levels` (assoc_level_maps(L) maps per batch row and element).
size_t assoc_level_maps(int L);
hipError_t launch_samu_baseline(int variant, const SamuParams& p, const float* ctl, const float* mtab,
                                float* levels, void* y, int y_f32, float* z_final, hipStream_t s);
hipError_t launch_rglru_baseline(int variant, const RglruParams& p, float* levels, void* y, int y_f32,
                                 float* h_final, hipStream_t s);

// ------------------------------------------------ RG-LRU gate projections ---
// 16-block block-diagonal projections x -> l^x, l^a (BF16) and their adjoint;
// dw_part / db_part: gate_proj_ranges(BL) x [2][16][Db][Db] / [2][D] floats.
int gate_proj_ranges(int BL);
hipError_t launch_gate_proj_fwd(int BL, int D, const void* x, const void* w_x, const float* b_x,
                                const void* w_a, const float* b_a, void* lx, void* la, hipStream_t s);
hipError_t launch_gate_proj_bwd(int BL, int D, const void* x, const void* w_x, const void* w_a, const void* dlx,
                                const void* dla, int f32, const void* dx_in, void* dx_out, float* dw_x,
                                float* db_x, float* dw_a, float* db_a, float* dw_part, float* db_part,
                                hipStream_t s);

}  // namespace lrs
