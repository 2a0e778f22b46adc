/*
 * samu_scan.h -- C ABI of the MI355X (gfx950) exact chunked affine scans:
 * the SAMU complex diagonal recurrence and the RG-LRU real gated recurrence,
 * forward and backward.
 *
 * Sources: page "SAMU 与 RG-LRU 的 H800 训练性能对比" (section 02 for the
 * shapes B, L, D, K and the forward/backward scopes; section 04 for RG-LRU;
 * section 05 for SAMU), page "SAMU strengthened-baseline H800 report"
 * ("Reverse complex backward"; "Memory, scratch, parameters, and launches"),
 * page "Griffin 第 4、5 节 H800 对照协议" ("RG-LRU 的固定方程", "SAMU 的固定方程").
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers on the current HIP device, 16-byte
 *     aligned, densely packed row-major in the shapes given.  BF16 tensors
 *     hold IEEE bfloat16 bit patterns; complex tensors interleave (Re, Im).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns after enqueueing.  All arguments are
 *     validated before the first enqueue: any status other than SCAN_OK means
 *     nothing was enqueued, except SCAN_ERR_DEVICE, which reports a failed
 *     launch (scan_last_error() then carries the HIP error text).
 *   - The library allocates no device memory and keeps no pointer after a
 *     call returns.  The caller owns every buffer.  `saved` is written by the
 *     forward call and read by the backward call of the same shape (B, L, D,
 *     K); it must be left untouched in between.  `workspace` contents are
 *     undefined after a call; concurrent calls need distinct workspaces.
 *   - Gradients overwrite their buffers.  Outputs must not overlap inputs
 *     (SCAN_ERR_ALIAS).
 *   - Results are bitwise deterministic for the same inputs, (K, G), device
 *     and library build: every reduction has a fixed order and nothing is
 *     accumulated atomically.  (The SAMU single-pass scans hand states
 *     between workgroups through atomic loads and stores of whole words, in
 *     an order of evaluation fixed by the group index alone.)
 *   - K (chunk length) is 16 or 32.  G (chunks per group of the two-level
 *     prefix) is >= 1, or 0 for the library's choice.
 *       SAMU: G = 0 means groups of 8 chunks.  Any G <= 16 runs the
 *       single-pass scans (one workgroup per group of chunks forms the
 *       chunk summaries, takes the state entering its group from the
 *       earlier groups and replays, in one launch per direction); G > 16
 *       runs separate summary, three-launch prefix (compose U_g, scan over
 *       groups, chunk entries) and replay launches.
 *       RG-LRU: G = 0 means the serial prefix when ceil(L/K) <= 128, else
 *       groups of max(16, ceil(ceil(L/K) / 128)) chunks.
 *     G >= ceil(L/K) gives a single group (the serial chunk-to-chunk
 *     prefix).  The forward and backward calls may use different G (e.g. a
 *     serial forward prefix with a grouped reverse prefix): the grouping
 *     changes only the parenthesization of an exact composition.
 *   - B >= 1, L >= 1 with any remainder (the last chunk has L - (C-1) K
 *     tokens), ceil(L/K) <= 65535, B <= 65535, B*L < 2^31.
 */
#ifndef SAMU_SCAN_H
#define SAMU_SCAN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int scan_status;
enum {
    SCAN_OK = 0,
    SCAN_ERR_NULL = -1,       /* a required pointer is NULL */
    SCAN_ERR_SHAPE = -2,      /* unsupported B, L, D, K, G or dtype code */
    SCAN_ERR_ALIGN = -3,      /* a pointer is not 16-byte aligned */
    SCAN_ERR_WORKSPACE = -4,  /* workspace_bytes below the size query */
    SCAN_ERR_DEVICE = -5,     /* a kernel launch failed */
    SCAN_ERR_ALIAS = -6       /* an output overlaps an input or another output */
};

/* Element type of the visible output y and of the input gradients. */
enum { SCAN_BF16 = 0, SCAN_F32 = 1 };

/* Text of the last non-OK status returned on the calling thread. */
const char* scan_last_error(void);

/* ======================================================================
 * SAMU mixer scan (page "SAMU 与 RG-LRU 的 H800 训练性能对比", section 05).
 * D real state channels = M = D/2 complex modes; D must be a multiple of 8,
 * at most 1048576 (every call taking D rejects a wider state).
 *
 * Forward, per batch row and token t = 1..L:
 *   x~_t = [x_sel_t; 1], w^ = w / ||w||_2 (norm over all D+1 entries),
 *   p_t = tanh(x~_t . w^_phi), r_t = tanh(x~_t . w^_r), q = r / (1 + r^2),
 *   d_t = tanh(a_phi)/sqrt(M) p_t, c_t = tanh(a_r)/sqrt(M) q(r_t),
 *   E_t = e^{c_t}, C_t = cos d_t, S_t = sin d_t (once per token),
 *   lambda_{t,m} = e^{-nu_m E_t} [(cos th_m C_t - sin th_m S_t)
 *                                 + i (sin th_m C_t + cos th_m S_t)],
 *   z_{t,m} = lambda_{t,m} z_{t-1,m} + b_{t,m},   y_t = z_t,
 * computed as K-step chunk summaries, the grouped prefix Q_c = L_c o O_g and
 * an in-register replay.  y carries no write normalization.
 * ====================================================================== */

/* Bytes of the forward-to-backward record: p, r, the per-token special
 * functions, the mode table, the direction norms (1/||w|| and the FP64
 * squared norms), the entry state of every chunk and, for K = 32,
 * the state entering the second 16-token half of every chunk (the backward
 * replay starts its sub-chunks from these instead of recomputing them).
 * Independent of G, so a backward may use another grouping than its forward. */
size_t samu_scan_saved_bytes(int B, int L, int D, int K);

/* Workspace bytes of samu_scan_fwd (backward = 0) or samu_scan_bwd
 * (backward = 1).  Returns 0 for an unsupported shape. */
size_t samu_scan_workspace_bytes(int B, int L, int D, int K, int G, int backward);

/* The pages' analytical prefix scratch: 12 B per real channel per chunk
 * summary and per group summary, 12 B * B * D * (ceil(L/K) + groups), with no
 * group term for the serial prefix (page "SAMU strengthened-baseline H800
 * report", "Memory, scratch, parameters, and launches").  Same formula for
 * both scans. */
size_t scan_prefix_scratch_bytes(int B, int L, int D, int K, int G, int rglru);

/* Forward.
 *   x_sel   bf16 [B, L, D]         selector input
 *   b       bf16 [B, L, M, 2]      complex drive (Re, Im)
 *   w_phi, w_r  f32 [D+1]          direction vectors (last entry: the bias slot)
 *   a_phi, a_r  f32 [1]            signed amplitudes
 *   nu, theta   f32 [M]            static spectrum
 *   z0      f32 [B, M, 2] or NULL  initial state (NULL = 0)
 *   y       [B, L, M, 2] of y_dtype (SCAN_BF16: round-to-nearest-even of the
 *           FP32 state; SCAN_F32: the FP32 state)
 *   z_final f32 [B, M, 2] or NULL  state after the last token
 *   saved   samu_scan_saved_bytes() bytes, 16-byte aligned (written)
 *   workspace  samu_scan_workspace_bytes(..., 0) bytes */
scan_status samu_scan_fwd(int B, int L, int D, int K, int G,
                          const void* x_sel, const void* b,
                          const float* w_phi, const float* w_r,
                          const float* a_phi, const float* a_r,
                          const float* nu, const float* theta, const float* z0,
                          void* y, int y_dtype, float* z_final,
                          void* saved, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Backward: the exact adjoint (page section 05, 'backward'; page "SAMU
 * strengthened-baseline H800 report", "Reverse complex backward").  With
 * the cotangent convention dL/dRe + i dL/dIm,
 *   z-bar_{t-1} += conj(lambda_t) z-bar_t, b-bar_t = z-bar_t,
 *   gamma = conj(lambda_t) z-bar_t conj(z_{t-1}):
 *   d nu_m = -sum_t E_t Re gamma, d theta_m = sum_t Im gamma,
 *   c-bar_t = -E_t sum_m nu_m Re gamma, d-bar_t = sum_m Im gamma
 *   (per 64-mode tile, then a fixed-order second stage),
 *   p-bar = d-bar tanh(a_phi)/sqrt(M), r-bar = c-bar tanh(a_r)/sqrt(M)
 *           (1 - r^2)/(1 + r^2)^2,
 *   dx_sel = u_phi w^_phi + u_r w^_r with u = p-bar (1 - p^2), r-bar (1 - r^2),
 *   dw = (g - w^ (w^ . g)) / ||w|| with g = sum_t u_t x~_t,
 *   da_phi = (1 - tanh^2 a_phi)/sqrt(M) sum_t d-bar_t p_t (da_r with c-bar q).
 *   x_sel, b, parameters: as passed to samu_scan_fwd
 *   saved    the record written by samu_scan_fwd
 *   dy       bf16 [B, L, M, 2]      dense output cotangent
 *   dz_final f32 [B, M, 2] or NULL  cotangent of z_final (NULL = 0)
 *   dx_sel   [B, L, D] of grad_dtype;  db  [B, L, M, 2] of grad_dtype
 *   dz0      f32 [B, M, 2] or NULL  gradient of the initial state
 *   dw_phi, dw_r f32 [D+1]; da_phi, da_r f32 [1]; dnu, dtheta f32 [M]
 *   workspace  samu_scan_workspace_bytes(..., 1) bytes */
scan_status samu_scan_bwd(int B, int L, int D, int K, int G,
                          const void* x_sel, const void* b,
                          const float* w_phi, const float* w_r,
                          const float* a_phi, const float* a_r,
                          const float* nu, const float* theta,
                          const void* saved, const void* dy, const float* dz_final,
                          void* dx_sel, void* db, int grad_dtype, float* dz0,
                          float* dw_phi, float* dw_r, float* da_phi, float* da_r,
                          float* dnu, float* dtheta,
                          void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as samu_scan_fwd, with the same arguments except the workspace,
 * which this call takes from a static device array of
 * SAMU_SCAN_NOALLOC_SCRATCH_BYTES bytes that each device holds until the
 * process ends.  The call allocates nothing.  A shape whose forward workspace
 * (samu_scan_workspace_bytes(..., 0)) exceeds that size returns
 * SCAN_ERR_WORKSPACE before anything is enqueued.  All calls on one device
 * share its array: calls that overlap in time on one device (on two streams
 * or from two threads) race on it and must be serialized by the caller.
 * The caller still provides y, z_final and the saved record. */
#define SAMU_SCAN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
scan_status samu_scan_fwd_noalloc(int B, int L, int D, int K, int G,
                                  const void* x_sel, const void* b,
                                  const float* w_phi, const float* w_r,
                                  const float* a_phi, const float* a_r,
                                  const float* nu, const float* theta, const float* z0,
                                  void* y, int y_dtype, float* z_final, void* saved,
                                  void* stream);

/* One generation step for B sequences in a single launch (page "Griffin 第
 * 4、5 节 H800 对照协议", "SAMU 的固定方程": control projection, transition
 * rebuild, FP32 state update and BF16 output in one kernel; equations of
 * page "SAMU 与 RG-LRU 的 H800 训练性能对比", section 05, at one token):
 *   z_out = lambda(x_sel) z_in + b,  y = z_out.
 *   x_sel   bf16 [B, D]            selector of the new token
 *   b       bf16 [B, M, 2]         complex drive of the new token
 *   w_phi, w_r, a_phi, a_r, nu, theta  as for samu_scan_fwd
 *   z_in    f32 [B, M, 2] or NULL  state before the token (NULL = 0)
 *   table   samu_scan_decode_table_bytes(D) bytes written by
 *           samu_scan_decode_prepare for these parameters, or
 *           NULL: the step then forms the per-mode phasors (in FP64) and the
 *           direction norms itself, every call
 *   z_out   f32 [B, M, 2]          state after the token; may equal z_in
 *                                  (updated in place), must not overlap it
 *                                  otherwise
 *   y       [B, M, 2] of y_dtype   output of the token
 * Needs 1 <= B <= 65535 and D as for samu_scan_fwd; allocates nothing. */
scan_status samu_scan_decode(int B, int D, const void* x_sel, const void* b,
                             const float* w_phi, const float* w_r,
                             const float* a_phi, const float* a_r,
                             const float* nu, const float* theta, const void* table,
                             const float* z_in, float* z_out, void* y, int y_dtype,
                             void* stream);

/* The per-parameter constants of the decode step, formed once for a set of
 * parameters and reused by every step: for each mode the phasor e^{i theta}
 * (an FP32 hi + lo pair from an FP64 evaluation) and -nu log2(e); 1/||w|| of
 * both directions (norm over all D+1 entries) and tanh(a)/sqrt(M) of both
 * amplitudes.  The table is caller-owned, 16-byte aligned,
 * samu_scan_decode_table_bytes(D) bytes (0 = unsupported D); it must be
 * prepared again when a parameter changes. */
size_t samu_scan_decode_table_bytes(int D);
scan_status samu_scan_decode_prepare(int D, const float* w_phi, const float* w_r,
                                     const float* a_phi, const float* a_r,
                                     const float* nu, const float* theta,
                                     void* table, void* stream);

/* ======================================================================
 * RG-LRU scan (page "SAMU 与 RG-LRU 的 H800 训练性能对比", section 04; reset
 * semantics also page "Griffin 第 4、5 节 H800 对照协议", "RG-LRU 的固定方程").
 * D real channels, D even, at most 1048576.
 *   g^x = sigmoid(l^x), g^a = sigmoid(l^a), a_t = exp(-8 g^a softplus(alpha)),
 *   b_t = x_t g^x sqrt(max(1 - a_t^2, 0)),  h_t = a_t h_{t-1} + b_t,  y_t = h_t;
 *   at a segment start (reset[b, t] != 0): a_t = 0 and the multiplier is 1.
 * K and G as for SAMU; G = 0 picks groups of 8 chunks at K = 16 and the
 * pages' long groups at K = 32.  At K = 16 with G <= 16 each direction is
 * one single-pass launch (after a small one that clears its hand-off words),
 * as for SAMU; otherwise the three-launch prefix runs.  Either way nothing
 * is accumulated atomically and results are bitwise reproducible for the
 * same inputs, K, G and device.
 * ====================================================================== */

size_t rglru_scan_saved_bytes(int B, int L, int D, int K);
size_t rglru_scan_workspace_bytes(int B, int L, int D, int K, int G, int backward);

/* Forward.
 *   x, lx, la  bf16 [B, L, D]     input and the two gate logits
 *   alpha      f32 [D]            static retention parameter
 *   reset      uint8 [B, L] or NULL (0/1 segment-start flags; NULL = none)
 *   h0         f32 [B, D] or NULL  initial state (NULL = 0)
 *   y          [B, L, D] of y_dtype; h_final f32 [B, D] or NULL
 *   saved      rglru_scan_saved_bytes() bytes (written) */
scan_status rglru_scan_fwd(int B, int L, int D, int K, int G,
                           const void* x, const void* lx, const void* la,
                           const float* alpha, const unsigned char* reset,
                           const float* h0, void* y, int y_dtype, float* h_final,
                           void* saved, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Backward: reverse real affine scan with resets as a = 0, gates recomputed;
 * the square-root derivative d sqrt(u)/du is capped at 1000.
 *   dy        bf16 [B, L, D];  dh_final f32 [B, D] or NULL (= 0)
 *   dx, dlx, dla  [B, L, D] of grad_dtype (dla = 0 at segment starts)
 *   dalpha    f32 [D], summed over batch rows and chunks
 *   dh0       f32 [B, D] or NULL */
scan_status rglru_scan_bwd(int B, int L, int D, int K, int G,
                           const void* x, const void* lx, const void* la,
                           const float* alpha, const unsigned char* reset,
                           const void* saved, const void* dy, const float* dh_final,
                           void* dx, void* dlx, void* dla, int grad_dtype,
                           float* dalpha, float* dh0,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * RG-LRU gate projections (page "Griffin 第 4、5 节 H800 对照协议",
 * "RG-LRU 的固定方程": both gates come from 16-block block-diagonal linear
 * layers).  With Db = D/16 and block i covering channels [i Db, (i+1) Db):
 *   l[t, i Db + o] = b[i Db + o] + sum_k W[i][o][k] x[t, i Db + k],
 * for (l^x; W_x, b_x) and (l^a; W_a, b_a).  BF16 matrix-core products with
 * FP32 accumulation; the logits are rounded to BF16 (nearest even), the
 * input format of rglru_scan_fwd.  Needs D a multiple of 256, D <= 2560.
 *   x         bf16 [B, L, D]
 *   w_x, w_a  bf16 [16, D/16, D/16]  (block, output, input)
 *   b_x, b_a  f32 [D]
 *   lx, la    bf16 [B, L, D]        (written) */
scan_status rglru_gate_proj_fwd(int B, int L, int D, const void* x,
                                const void* w_x, const float* b_x,
                                const void* w_a, const float* b_a,
                                void* lx, void* la, void* stream);

/* Adjoint of the projections for the logit cotangents dlx, dla (as written
 * by rglru_scan_bwd, of grad_dtype); with BF16 cotangents and D <= 2048 one
 * pass over the tensors forms dx and the weight partials together:
 *   dx_out = dx_in + per block W_x^T dlx + W_a^T dla   ([B, L, D], grad_dtype;
 *            dx_out may equal dx_in, must not overlap it otherwise),
 *   dw = sum_t dl x^T per block (f32 [16, D/16, D/16]), db = sum_t dl (f32 [D]).
 * SCAN_F32 cotangents are split exactly into three BF16 terms (hi + mid +
 * lo), each multiplied on the BF16 matrix cores with FP32 accumulation --
 * the same exact products as FP32 multiplies.  The token sums for dw and db
 * are split over fixed ranges of 2048 tokens, whose FP32 partials (in the
 * caller's workspace, rglru_gate_proj_bwd_workspace_bytes bytes) are added
 * in range order in FP64: results are bitwise reproducible.  Errors as for
 * the scans: shape, dtype code, NULL, alignment, aliasing and workspace size
 * are checked before anything is queued. */
size_t rglru_gate_proj_bwd_workspace_bytes(int B, int L, int D);
scan_status rglru_gate_proj_bwd(int B, int L, int D, const void* x,
                                const void* w_x, const void* w_a,
                                const void* dlx, const void* dla, int grad_dtype,
                                const void* dx_in, void* dx_out,
                                float* dw_x, float* db_x, float* dw_a, float* db_a,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * Comparison scans of the scan-latency experiment (page "Griffin 第 4、5 节
 * H800 对照协议", experiment-coverage matrix, the Fig. 8(a) row: the exact
 * chunked scan against a per-channel on-chip sequential scan and
 * associative scans, for SAMU and RG-LRU).  Forward only; same equations,
 * arguments and output conventions as samu_scan_fwd / rglru_scan_fwd.
 *   SCAN_BASELINE_SEQUENTIAL   one lane per (batch row, mode or channel)
 *                              walks all L tokens in order;
 *   SCAN_BASELINE_ASSOCIATIVE  the recursive pairwise (log-depth) scan:
 *                              log2(L) reduce and log2(L) expand passes over
 *                              HBM level arrays held in the workspace.
 * These are baselines for measurement, not the fast path.
 * ====================================================================== */
typedef enum {
    SCAN_BASELINE_SEQUENTIAL = 0,
    SCAN_BASELINE_ASSOCIATIVE = 1
} scan_baseline;

/* Workspace bytes (0 = unsupported variant or shape; the RG-LRU sequential
 * scan needs none).  The SAMU workspace holds the controller's per-token
 * record and the mode table as well. */
size_t samu_scan_baseline_workspace_bytes(int variant, int B, int L, int D);
size_t rglru_scan_baseline_workspace_bytes(int variant, int B, int L, int D);

scan_status samu_scan_baseline_fwd(int variant, int B, int L, int D,
                                   const void* x_sel, const void* b,
                                   const float* w_phi, const float* w_r,
                                   const float* a_phi, const float* a_r,
                                   const float* nu, const float* theta, const float* z0,
                                   void* y, int y_dtype, float* z_final,
                                   void* workspace, size_t workspace_bytes, void* stream);
scan_status rglru_scan_baseline_fwd(int variant, int B, int L, int D,
                                    const void* x, const void* lx, const void* la,
                                    const float* alpha, const unsigned char* reset,
                                    const float* h0, void* y, int y_dtype, float* h_final,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================
 * Per-kernel timing (page "SAMU 与 RG-LRU 的 H800 训练性能对比", section 05,
 * the backward component times; section 06 and page "SAMU
 * strengthened-baseline H800 report" count kernel launches per F+B).
 * While enabled, every kernel launched by this library is bracketed by two
 * HIP events on its stream.  Not thread-safe against concurrent enqueues.
 * ====================================================================== */
void scan_profile_enable(int on);
/* Number of kernel kinds (ids 0 .. n-1) and the name of each. */
int scan_profile_kernel_count(void);
const char* scan_profile_kernel_name(int id);
/* Waits for every recorded event, writes per-kernel total milliseconds and
 * launch counts (arrays of scan_profile_kernel_count() entries; either may be
 * NULL), then forgets the records.  Returns SCAN_OK or SCAN_ERR_DEVICE. */
scan_status scan_profile_collect(double* total_ms, int* launches);

/* ======================================================================
 * Hand-off wait limit of the single-pass scans (SAMU forward and backward;
 * RG-LRU forward and backward at K=16 with groups of at most 16 chunks).
 * A workgroup of these scans waits for words that earlier workgroups of the
 * same launch publish; every such wait is bounded by a number of polls.  A
 * wait that expires yields NaN, which reaches every output downstream of
 * it, instead of a plausible wrong value.  The default (16384 polls) is far
 * above what a wait takes while the publishing workgroup runs; the limit
 * exists so that tests can force the expiry path.
 * Sets the limit for launches enqueued from now on (polls >= 0; a negative
 * value restores the default) and returns the previous limit.  Process-wide;
 * launches already captured into a graph keep the limit they were enqueued
 * with.
 * ====================================================================== */
int scan_set_handoff_poll_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* SAMU_SCAN_H */
