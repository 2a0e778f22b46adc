// capi.cpp -- the C ABI: argument validation, buffer layout inside the
// caller's saved/workspace memory, kernel sequencing, error text and the
// per-kernel event profiler.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"
#include "samu_scan.h"

namespace lrs {

// ------------------------------------------------------------- errors ---
static thread_local std::string g_last_error;

static scan_status fail(scan_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

scan_status set_last_error(scan_status st, const char* msg) { return fail(st, msg); }

// ------------------------------------------------- hand-off wait limit ---
std::atomic<int> g_handoff_polls{HANDOFF_POLLS_DEFAULT};
int handoff_poll_limit() { return g_handoff_polls.load(std::memory_order_relaxed); }

// ----------------------------------------------------------- profiler ---
namespace {
struct ProfRecord {
    int id;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_prof_pool;
hipEvent_t g_prof_pending = nullptr;
int g_prof_pending_id = -1;

hipEvent_t pool_get() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

static const char* const kKernelNames[K_NUM_KERNELS] = {
    "samu_controller", "samu_chunk_summary", "prefix_group_compose", "prefix_group_scan",
    "prefix_chunk_entries", "samu_replay", "samu_reverse_summary", "samu_bwd_replay",
    "samu_controller_bwd", "samu_params", "rglru_chunk_summary", "rglru_replay",
    "rglru_reverse_summary", "rglru_bwd_replay", "rglru_alpha", "samu_decode",
    "baseline_sequential", "baseline_associative", "gate_projection", "gate_projection_dx",
    "gate_projection_dw", "gate_projection_reduce", "samu_forward_scan", "samu_backward_scan", "clear",
    "gate_projection_adjoint", "rglru_forward_scan", "rglru_backward_scan"};

const char* kernel_name(int id) { return (id >= 0 && id < K_NUM_KERNELS) ? kKernelNames[id] : "?"; }

bool profiler_enabled() { return g_prof_on; }

void profiler_before(int id, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending = pool_get();
    g_prof_pending_id = id;
    if (g_prof_pending) (void)hipEventRecord(g_prof_pending, s);
}

void profiler_after(int id, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t a = g_prof_pending;
    g_prof_pending = nullptr;
    if (!a || g_prof_pending_id != id) return;
    hipEvent_t b = pool_get();
    if (!b) { g_prof_pool.push_back(a); return; }
    (void)hipEventRecord(b, s);
    g_prof_records.push_back({id, a, b});
}

// -------------------------------------------------------------- sizes ---
static constexpr size_t kAlign = 256;
static size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over a caller-owned base pointer (or a null base for sizing).
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off = align_up(off + count * sizeof(T));
        return p;
    }
};

// G == 0 picks the grouping from the shape (measured on MI355X at the
// pages' workloads, F+B at B = 1 and 8, D = 1024..2560, L = 2K..131K):
//   * at most kSerialMaxChunks chunks per row: the serial prefix (one group;
//     one launch per direction instead of three, and the walk is short);
//   * otherwise about kTargetGroups groups per row, each at least
//     min_group chunks long (8 for the complex scan, 16 for the real one).
static constexpr int64_t kSerialMaxChunks = 128;
static constexpr int64_t kTargetGroups = 128;
static bool chunking(int B, int L, int K, int G, int min_group, Chunking* ch, int default_group = 0) {
    if (B < 1 || L < 1 || B > 65535 || (K != 16 && K != 32) || G < 0) return false;
    const int64_t C = ceil_div(L, K);
    if (C > 65535 || (int64_t)B * L > 0x7fffffff) return false;
    int64_t g = G;
    if (g == 0 && default_group > 0) g = default_group;
    if (g == 0) g = C <= kSerialMaxChunks ? C : std::max<int64_t>(min_group, ceil_div(C, kTargetGroups));
    ch->B = B;
    ch->L = L;
    ch->K = K;
    ch->C = (int)C;
    ch->G = (int)std::min<int64_t>(g, C);
    ch->NG = (int)ceil_div(C, ch->G);
    return true;
}

static constexpr int kSamuMinGroup = 8;      // see chunking()
static constexpr int kRglruMinGroup = 16;
// RG-LRU with K = 16 and G == 0: groups of kRglruGroup chunks on the
// single-pass path (rglru_fused); K = 32 and longer groups take the
// three-kernel prefix.
static constexpr int kRglruGroup = 8;
// SAMU with G == 0: groups of kSamuGroup chunks on the grouped path (one
// workgroup per group; see launch_samu_gscan), which any G up to
// SAMU_GROUP_MAX takes; longer groups take the three-kernel prefix.
static constexpr int kSamuGroup = 8;
static bool samu_fused(const Chunking& ch) { return ch.G <= SAMU_GROUP_MAX; }

struct SamuSaved {
    float *p, *r, *u, *ctl, *mtab, *inv_norm, *entries, *mid, *crec;
};
static SamuSaved samu_saved_layout(void* base, const Chunking& ch, int M, size_t* bytes) {
    Carver cv(base);
    SamuSaved s;
    const size_t BL = (size_t)ch.B * ch.L;
    s.p = cv.take<float>(BL);
    s.r = cv.take<float>(BL);
    s.u = cv.take<float>(BL * 2);
    s.ctl = cv.take<float>(BL * 4);
    s.mtab = cv.take<float>((size_t)M * 16);
    s.inv_norm = cv.take<float>(8);  // 1/||w_phi||, 1/||w_r||, pad, then the FP64 squared norms
    s.entries = cv.take<float>((size_t)ch.B * ch.C * M * 2);
    s.mid = cv.take<float>((size_t)ch.B * ch.C * samu_mid_states(ch.K) * M * 2);
    s.crec = cv.take<float>((size_t)ch.B * ch.C * 4);  // (G_c, cos D_c, sin D_c, 0) per chunk
    if (bytes) *bytes = cv.off;
    return s;
}

// The grouped path needs only the single-pass forward's hand-off words; the
// three-kernel prefix keeps chunk summaries, records and group summaries.
struct SamuFwdWs {
    float *summ, *chunk, *gsum;
    void* pub;
    size_t pub_bytes;
};
static SamuFwdWs samu_fwd_ws_layout(void* base, const Chunking& ch, int M, size_t* bytes) {
    Carver cv(base);
    SamuFwdWs w{};
    if (samu_fused(ch)) {
        w.pub_bytes = samu_gscan_pub_bytes(ch, M);
        w.pub = cv.take<uint64_t>(w.pub_bytes / sizeof(uint64_t));
    } else {
        w.summ = cv.take<float>((size_t)ch.B * ch.C * M * 2);
        w.chunk = cv.take<float>((size_t)ch.B * ch.C * 4);
        w.gsum = cv.take<float>((size_t)ch.B * ch.NG * M * 6);
    }
    if (bytes) *bytes = cv.off;
    return w;
}

// The grouped path keeps its reverse summaries and carries in LDS and needs
// only the single-pass backward's hand-off words and one (d nu, d theta) row
// per group; the three-kernel prefix keeps summaries, carries and one row
// per chunk.
struct SamuBwdWs {
    float *rsumm, *rchunk, *rgsum, *carry, *tok_part, *mode_part, *g_part;
    void* pub;
    size_t pub_bytes;
    int n_tiles, n_blk;
};
static SamuBwdWs samu_bwd_ws_layout(void* base, const Chunking& ch, int D, int M, size_t* bytes) {
    Carver cv(base);
    SamuBwdWs w{};
    const size_t BCM = (size_t)ch.B * ch.C * M;
    w.n_tiles = samu_bwd_tiles(M);
    w.n_blk = (int)ceil_div((int64_t)ch.B * ch.L, samu_ctl_tok_per_blk());
    const bool fused = samu_fused(ch);
    if (fused) {
        w.pub_bytes = samu_gscan_pub_bytes(ch, M);
        w.pub = cv.take<uint64_t>(w.pub_bytes / sizeof(uint64_t));
    } else {
        w.rsumm = cv.take<float>(BCM * 2);
        w.rchunk = cv.take<float>((size_t)ch.B * ch.C * 4);
        w.rgsum = cv.take<float>((size_t)ch.B * ch.NG * M * 6);
        w.carry = cv.take<float>(BCM * 2);
    }
    w.tok_part = cv.take<float>((size_t)ch.B * w.n_tiles * ch.L * 2);
    w.mode_part = cv.take<float>((size_t)ch.B * (fused ? ch.NG : ch.C) * M * 2);
    w.g_part = cv.take<float>((size_t)w.n_blk * samu_param_columns(D) * 2);
    if (bytes) *bytes = cv.off;
    return w;
}

struct RgSaved {
    float* entries;
};
static RgSaved rg_saved_layout(void* base, const Chunking& ch, int D, size_t* bytes) {
    Carver cv(base);
    RgSaved s;
    s.entries = cv.take<float>((size_t)ch.B * ch.C * D);
    if (bytes) *bytes = cv.off;
    return s;
}

// The single-pass path (rglru_fused) needs only its hand-off words and, in
// the backward, one alpha row per group; the three-kernel prefix keeps chunk
// summaries, group summaries, carries and one alpha row per chunk.
struct RgWs {
    float *summ, *gsum, *carry, *alpha_part;
    void* pub;
    size_t pub_bytes;
    int alpha_rows;
};
static RgWs rg_ws_layout(void* base, const Chunking& ch, int D, bool backward, size_t* bytes) {
    Carver cv(base);
    RgWs w{};
    const size_t BCD = (size_t)ch.B * ch.C * D;
    if (rglru_fused(ch)) {
        w.pub_bytes = rglru_pub_bytes(ch, D);
        w.pub = cv.take<uint64_t>(w.pub_bytes / sizeof(uint64_t));
        w.alpha_rows = ch.B * ch.NG;
    } else {
        w.summ = cv.take<float>(BCD * 2);
        w.gsum = cv.take<float>((size_t)ch.B * ch.NG * D * 3);
        if (backward) w.carry = cv.take<float>(BCD);
        w.alpha_rows = ch.B * ch.C;
    }
    if (backward) w.alpha_part = cv.take<float>((size_t)w.alpha_rows * D);
    if (bytes) *bytes = cv.off;
    return w;
}

// --------------------------------------------------------- validation ---
struct Span {
    const void* p;
    size_t n;
    const char* name;
};

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static scan_status check_ptrs(std::initializer_list<Span> req, std::initializer_list<Span> opt) {
    for (const Span& s : req) {
        if (!s.p) return fail(SCAN_ERR_NULL, std::string(s.name) + " is NULL");
        if (!aligned16(s.p)) return fail(SCAN_ERR_ALIGN, std::string(s.name) + " is not 16-byte aligned");
    }
    for (const Span& s : opt)
        if (s.p && !aligned16(s.p)) return fail(SCAN_ERR_ALIGN, std::string(s.name) + " is not 16-byte aligned");
    return SCAN_OK;
}

static bool overlap(const Span& a, const Span& b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// outputs must not overlap inputs nor each other
static scan_status check_alias(const std::vector<Span>& ins, const std::vector<Span>& outs) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in))
                return fail(SCAN_ERR_ALIAS, std::string(outs[i].name) + " overlaps " + in.name);
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlap(outs[i], outs[j]))
                return fail(SCAN_ERR_ALIAS, std::string(outs[i].name) + " overlaps " + outs[j].name);
    }
    return SCAN_OK;
}

static scan_status device_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return SCAN_OK;
    return fail(SCAN_ERR_DEVICE, std::string(where) + ": " + hipGetErrorString(e));
}

#define LRS_TRY(expr, where)                                    \
    do {                                                        \
        scan_status _st = device_status((expr), (where));       \
        if (_st != SCAN_OK) return _st;                         \
    } while (0)

// Widest state accepted: keeps every chunk's rows (at most 32 tokens of
// 8-byte elements) far inside the 32-bit byte ranges of the kernels' buffer
// descriptors and offsets.
static constexpr int kMaxD = 1 << 20;

static bool samu_shape(int B, int L, int D, int K, int G, Chunking* ch) {
    if (D < 8 || D % 8 != 0 || D > kMaxD) return false;
    return chunking(B, L, K, G, kSamuMinGroup, ch, kSamuGroup);
}

static bool rglru_shape(int B, int L, int D, int K, int G, Chunking* ch) {
    if (D < 2 || D % 2 != 0 || D > kMaxD) return false;
    return chunking(B, L, K, G, kRglruMinGroup, ch, K == 16 ? kRglruGroup : 0);
}

static std::string shape_text(int B, int L, int D, int K, int G) {
    return "B=" + std::to_string(B) + " L=" + std::to_string(L) + " D=" + std::to_string(D) +
           " K=" + std::to_string(K) + " G=" + std::to_string(G);
}

}  // namespace lrs

using namespace lrs;

extern "C" {

const char* scan_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------- SAMU ---
size_t samu_scan_saved_bytes(int B, int L, int D, int K) {
    Chunking ch;
    if (!samu_shape(B, L, D, K, 0, &ch)) return 0;
    size_t n = 0;
    samu_saved_layout(nullptr, ch, D / 2, &n);
    return n;
}

size_t samu_scan_workspace_bytes(int B, int L, int D, int K, int G, int backward) {
    Chunking ch;
    if (!samu_shape(B, L, D, K, G, &ch)) return 0;
    size_t n = 0;
    if (backward) samu_bwd_ws_layout(nullptr, ch, D, D / 2, &n);
    else samu_fwd_ws_layout(nullptr, ch, D / 2, &n);
    return n;
}

size_t scan_prefix_scratch_bytes(int B, int L, int D, int K, int G, int rglru) {
    Chunking ch;
    const bool ok = rglru ? rglru_shape(B, L, D, K, G, &ch) : samu_shape(B, L, D, K, G, &ch);
    if (!ok) return 0;
    const size_t groups = ch.NG > 1 ? (size_t)ch.NG : 0;
    return (size_t)12 * B * D * ((size_t)ch.C + groups);
}

scan_status samu_scan_fwd(int B, int L, int D, int K, int G, const void* x_sel, const void* b,
                          const float* w_phi, const float* w_r, const float* a_phi, const float* a_r,
                          const float* nu, const float* theta, const float* z0, void* y, int y_dtype,
                          float* z_final, void* saved, void* workspace, size_t workspace_bytes,
                          void* stream) {
    Chunking ch;
    if (!samu_shape(B, L, D, K, G, &ch))
        return fail(SCAN_ERR_SHAPE, "samu_scan_fwd: unsupported shape " + shape_text(B, L, D, K, G) +
                                        " (need B, L >= 1, 8 <= D <= 1048576 a multiple of 8, K in {16, 32},"
                                        " G >= 0, ceil(L/K) <= 65535)");
    if (y_dtype != SCAN_BF16 && y_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "samu_scan_fwd: y_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs({{x_sel, 0, "x_sel"}, {b, 0, "b"}, {w_phi, 0, "w_phi"}, {w_r, 0, "w_r"},
                                 {a_phi, 0, "a_phi"}, {a_r, 0, "a_r"}, {nu, 0, "nu"}, {theta, 0, "theta"},
                                 {y, 0, "y"}, {saved, 0, "saved"}, {workspace, 0, "workspace"}},
                                {{z0, 0, "z0"}, {z_final, 0, "z_final"}});
    if (st != SCAN_OK) return st;
    const int M = D / 2;
    size_t need = 0, saved_n = 0;
    samu_fwd_ws_layout(nullptr, ch, M, &need);
    samu_saved_layout(nullptr, ch, M, &saved_n);
    if (workspace_bytes < need)
        return fail(SCAN_ERR_WORKSPACE, "samu_scan_fwd: workspace_bytes " + std::to_string(workspace_bytes) +
                                            " < " + std::to_string(need));
    const size_t BL = (size_t)B * L, BLM = BL * M;
    const size_t ysz = BLM * 2 * (y_dtype == SCAN_F32 ? 4 : 2);
    st = check_alias({{x_sel, BL * D * 2, "x_sel"}, {b, BLM * 4, "b"}, {w_phi, (size_t)(D + 1) * 4, "w_phi"},
                      {w_r, (size_t)(D + 1) * 4, "w_r"}, {a_phi, 4, "a_phi"}, {a_r, 4, "a_r"},
                      {nu, (size_t)M * 4, "nu"}, {theta, (size_t)M * 4, "theta"},
                      {z0, (size_t)B * M * 8, "z0"}},
                     {{y, ysz, "y"}, {z_final, (size_t)B * M * 8, "z_final"}, {saved, saved_n, "saved"},
                      {workspace, need, "workspace"}});
    if (st != SCAN_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    SamuParams p{B, L, D, M, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0};
    SamuSaved sv = samu_saved_layout(saved, ch, M, nullptr);
    SamuFwdWs ws = samu_fwd_ws_layout(workspace, ch, M, nullptr);
    // the controller also clears the single-pass forward's hand-off words
    LRS_TRY(launch_samu_controller(p, ch, sv.p, sv.r, sv.u, sv.ctl, sv.mtab, sv.inv_norm, sv.crec, ws.pub,
                                   ws.pub_bytes, s),
            "samu controller");
    if (samu_fused(ch)) {
        // summaries, U_g, the look-back over earlier groups and the replay,
        // in one launch
        LRS_TRY(launch_samu_gscan(p, ch, sv.ctl, sv.mtab, sv.crec, ws.pub, sv.entries, sv.mid, y,
                                  y_dtype == SCAN_F32, z_final, s),
                "samu forward scan");
        return SCAN_OK;
    }
    LRS_TRY(launch_samu_summary(p, ch, sv.ctl, sv.mtab, b, false, ws.summ, ws.chunk, s), "samu chunk summary");
    LRS_TRY(launch_prefix(2, false, ch, M, PrefixSummaries{nullptr, ws.summ, ws.chunk, sv.mtab}, ws.gsum, z0,
                          sv.entries, s),
            "samu prefix");
    LRS_TRY(launch_samu_replay(p, ch, sv.ctl, sv.mtab, sv.entries, sv.mid, y, y_dtype == SCAN_F32, z_final, s),
            "samu replay");
    return SCAN_OK;
}

scan_status samu_scan_bwd(int B, int L, int D, int K, int G, const void* x_sel, const void* b,
                          const float* w_phi, const float* w_r, const float* a_phi, const float* a_r,
                          const float* nu, const float* theta, const void* saved, const void* dy,
                          const float* dz_final, void* dx_sel, void* db, int grad_dtype, float* dz0,
                          float* dw_phi, float* dw_r, float* da_phi, float* da_r, float* dnu,
                          float* dtheta, void* workspace, size_t workspace_bytes, void* stream) {
    Chunking ch;
    if (!samu_shape(B, L, D, K, G, &ch))
        return fail(SCAN_ERR_SHAPE, "samu_scan_bwd: unsupported shape " + shape_text(B, L, D, K, G));
    if (grad_dtype != SCAN_BF16 && grad_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "samu_scan_bwd: grad_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs(
        {{x_sel, 0, "x_sel"}, {b, 0, "b"}, {w_phi, 0, "w_phi"}, {w_r, 0, "w_r"}, {a_phi, 0, "a_phi"},
         {a_r, 0, "a_r"}, {nu, 0, "nu"}, {theta, 0, "theta"}, {saved, 0, "saved"}, {dy, 0, "dy"},
         {dx_sel, 0, "dx_sel"}, {db, 0, "db"}, {dw_phi, 0, "dw_phi"}, {dw_r, 0, "dw_r"},
         {da_phi, 0, "da_phi"}, {da_r, 0, "da_r"}, {dnu, 0, "dnu"}, {dtheta, 0, "dtheta"},
         {workspace, 0, "workspace"}},
        {{dz_final, 0, "dz_final"}, {dz0, 0, "dz0"}});
    if (st != SCAN_OK) return st;
    const int M = D / 2;
    size_t need = 0, saved_n = 0;
    samu_bwd_ws_layout(nullptr, ch, D, M, &need);
    samu_saved_layout(nullptr, ch, M, &saved_n);
    if (workspace_bytes < need)
        return fail(SCAN_ERR_WORKSPACE, "samu_scan_bwd: workspace_bytes " + std::to_string(workspace_bytes) +
                                            " < " + std::to_string(need));
    const size_t BL = (size_t)B * L, BLM = BL * M;
    const size_t gsz = grad_dtype == SCAN_F32 ? 4 : 2;
    st = check_alias(
        {{x_sel, BL * D * 2, "x_sel"}, {b, BLM * 4, "b"}, {w_phi, (size_t)(D + 1) * 4, "w_phi"},
         {w_r, (size_t)(D + 1) * 4, "w_r"}, {a_phi, 4, "a_phi"}, {a_r, 4, "a_r"}, {nu, (size_t)M * 4, "nu"},
         {theta, (size_t)M * 4, "theta"}, {saved, saved_n, "saved"}, {dy, BLM * 4, "dy"},
         {dz_final, (size_t)B * M * 8, "dz_final"}},
        {{dx_sel, BL * D * gsz, "dx_sel"}, {db, BLM * 2 * gsz, "db"}, {dz0, (size_t)B * M * 8, "dz0"},
         {dw_phi, (size_t)(D + 1) * 4, "dw_phi"}, {dw_r, (size_t)(D + 1) * 4, "dw_r"}, {da_phi, 4, "da_phi"},
         {da_r, 4, "da_r"}, {dnu, (size_t)M * 4, "dnu"}, {dtheta, (size_t)M * 4, "dtheta"},
         {workspace, need, "workspace"}});
    if (st != SCAN_OK) return st;

    hipStream_t s = (hipStream_t)stream;
    SamuParams p{B, L, D, M, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, nullptr};
    SamuSaved sv = samu_saved_layout(const_cast<void*>(saved), ch, M, nullptr);
    SamuBwdWs ws = samu_bwd_ws_layout(workspace, ch, D, M, nullptr);
    const int f32 = grad_dtype == SCAN_F32;
    if (samu_fused(ch)) {
        // the hand-off words cleared, then reverse summaries, group carries
        // and the backward replay in one launch
        LRS_TRY(launch_samu_gbscan(p, ch, sv.ctl, sv.mtab, sv.entries, sv.mid, sv.crec, dz_final, ws.pub,
                                   ws.pub_bytes, dy, db, f32, dz0, ws.tok_part, ws.n_tiles, ws.mode_part, s),
                "samu backward scan");
    } else {
        LRS_TRY(launch_samu_summary(p, ch, sv.ctl, sv.mtab, dy, true, ws.rsumm, ws.rchunk, s),
                "samu reverse summary");
        LRS_TRY(launch_prefix(2, true, ch, M, PrefixSummaries{nullptr, ws.rsumm, ws.rchunk, sv.mtab}, ws.rgsum,
                              dz_final, ws.carry, s),
                "samu reverse prefix");
        LRS_TRY(launch_samu_bwd_replay(p, ch, sv.ctl, sv.mtab, sv.entries, sv.mid, ws.carry, dy, db, f32, dz0,
                                       ws.tok_part, ws.n_tiles, ws.mode_part, s),
                "samu backward replay");
    }
    LRS_TRY(launch_samu_ctl_bwd(p, sv.p, sv.r, sv.u, sv.inv_norm, ws.tok_part, ws.n_tiles, dx_sel, f32, ws.g_part, s),
            "samu controller backward");
    LRS_TRY(launch_samu_params(p, ch, reinterpret_cast<const double*>(sv.inv_norm + 4), ws.g_part, ws.n_blk,
                               ws.mode_part, samu_fused(ch) ? ch.B * ch.NG : ch.B * ch.C, dw_phi, dw_r, da_phi,
                               da_r, dnu, dtheta, s),
            "samu parameter reductions");
    return SCAN_OK;
}

// ---------------------------------------------------- comparison scans ---
struct SamuBaseWs {
    float *p, *r, *u, *ctl, *mtab, *levels;
};
static SamuBaseWs samu_base_layout(void* base, int B, int L, int M, int variant, size_t* bytes) {
    Carver cv(base);
    SamuBaseWs w{};
    const size_t BL = (size_t)B * L;
    w.p = cv.take<float>(BL);
    w.r = cv.take<float>(BL);
    w.u = cv.take<float>(BL * 2);
    w.ctl = cv.take<float>(BL * 4);
    w.mtab = cv.take<float>((size_t)M * 16);
    if (variant == SCAN_BASELINE_ASSOCIATIVE) w.levels = cv.take<float>(assoc_level_maps(L) * B * M * 4);
    if (bytes) *bytes = cv.off;
    return w;
}

static bool base_shape(int variant, int B, int L, int D, bool samu) {
    if (variant != SCAN_BASELINE_SEQUENTIAL && variant != SCAN_BASELINE_ASSOCIATIVE) return false;
    if (B < 1 || B > 65535 || L < 1 || (int64_t)B * L > 0x7fffffff) return false;
    if (D > kMaxD) return false;
    return samu ? (D >= 8 && D % 8 == 0) : (D >= 2 && D % 2 == 0);
}

size_t samu_scan_baseline_workspace_bytes(int variant, int B, int L, int D) {
    if (!base_shape(variant, B, L, D, true)) return 0;
    size_t n = 0;
    samu_base_layout(nullptr, B, L, D / 2, variant, &n);
    return n;
}

size_t rglru_scan_baseline_workspace_bytes(int variant, int B, int L, int D) {
    if (!base_shape(variant, B, L, D, false)) return 0;
    return variant == SCAN_BASELINE_ASSOCIATIVE ? assoc_level_maps(L) * B * D * 2 * sizeof(float) : 0;
}

scan_status samu_scan_baseline_fwd(int variant, int B, int L, int D, const void* x_sel, const void* b,
                                   const float* w_phi, const float* w_r, const float* a_phi,
                                   const float* a_r, const float* nu, const float* theta, const float* z0,
                                   void* y, int y_dtype, float* z_final, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!base_shape(variant, B, L, D, true))
        return fail(SCAN_ERR_SHAPE, "samu_scan_baseline_fwd: unsupported variant or shape B=" +
                                        std::to_string(B) + " L=" + std::to_string(L) + " D=" + std::to_string(D));
    if (y_dtype != SCAN_BF16 && y_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "samu_scan_baseline_fwd: y_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs({{x_sel, 0, "x_sel"}, {b, 0, "b"}, {w_phi, 0, "w_phi"}, {w_r, 0, "w_r"},
                                 {a_phi, 0, "a_phi"}, {a_r, 0, "a_r"}, {nu, 0, "nu"}, {theta, 0, "theta"},
                                 {y, 0, "y"}, {workspace, 0, "workspace"}},
                                {{z0, 0, "z0"}, {z_final, 0, "z_final"}});
    if (st != SCAN_OK) return st;
    const int M = D / 2;
    size_t need = 0;
    samu_base_layout(nullptr, B, L, M, variant, &need);
    if (workspace_bytes < need)
        return fail(SCAN_ERR_WORKSPACE, "samu_scan_baseline_fwd: workspace_bytes " +
                                            std::to_string(workspace_bytes) + " < " + std::to_string(need));
    const size_t BL = (size_t)B * L, BLM = BL * M;
    st = check_alias({{x_sel, BL * D * 2, "x_sel"}, {b, BLM * 4, "b"}, {w_phi, (size_t)(D + 1) * 4, "w_phi"},
                      {w_r, (size_t)(D + 1) * 4, "w_r"}, {a_phi, 4, "a_phi"}, {a_r, 4, "a_r"},
                      {nu, (size_t)M * 4, "nu"}, {theta, (size_t)M * 4, "theta"}, {z0, (size_t)B * M * 8, "z0"}},
                     {{y, BLM * 2 * (y_dtype == SCAN_F32 ? 4 : 2), "y"}, {z_final, (size_t)B * M * 8, "z_final"},
                      {workspace, need, "workspace"}});
    if (st != SCAN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    Chunking ch;
    chunking(B, L, 32, 0, kSamuMinGroup, &ch);  // the controller's chunk phasors are not used here
    SamuParams p{B, L, D, M, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0};
    SamuBaseWs ws = samu_base_layout(workspace, B, L, M, variant, nullptr);
    LRS_TRY(launch_samu_controller(p, ch, ws.p, ws.r, ws.u, ws.ctl, ws.mtab, nullptr, nullptr, nullptr, 0, s),
            "samu controller");
    LRS_TRY(launch_samu_baseline(variant, p, ws.ctl, ws.mtab, ws.levels, y, y_dtype == SCAN_F32, z_final, s),
            "samu comparison scan");
    return SCAN_OK;
}

scan_status rglru_scan_baseline_fwd(int variant, int B, int L, int D, const void* x, const void* lx,
                                    const void* la, const float* alpha, const unsigned char* reset,
                                    const float* h0, void* y, int y_dtype, float* h_final, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (!base_shape(variant, B, L, D, false))
        return fail(SCAN_ERR_SHAPE, "rglru_scan_baseline_fwd: unsupported variant or shape B=" +
                                        std::to_string(B) + " L=" + std::to_string(L) + " D=" + std::to_string(D));
    if (y_dtype != SCAN_BF16 && y_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "rglru_scan_baseline_fwd: y_dtype must be SCAN_BF16 or SCAN_F32");
    const size_t need = rglru_scan_baseline_workspace_bytes(variant, B, L, D);
    scan_status st = check_ptrs({{x, 0, "x"}, {lx, 0, "lx"}, {la, 0, "la"}, {alpha, 0, "alpha"}, {y, 0, "y"}},
                                {{h0, 0, "h0"}, {h_final, 0, "h_final"}, {workspace, 0, "workspace"}});
    if (st != SCAN_OK) return st;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SCAN_ERR_WORKSPACE, "rglru_scan_baseline_fwd: workspace_bytes " +
                                            std::to_string(workspace_bytes) + " < " + std::to_string(need));
    const size_t BL = (size_t)B * L, BLD = BL * D;
    st = check_alias({{x, BLD * 2, "x"}, {lx, BLD * 2, "lx"}, {la, BLD * 2, "la"}, {alpha, (size_t)D * 4, "alpha"},
                      {reset, BL, "reset"}, {h0, (size_t)B * D * 4, "h0"}},
                     {{y, BLD * (y_dtype == SCAN_F32 ? 4 : 2), "y"}, {h_final, (size_t)B * D * 4, "h_final"},
                      {need ? workspace : nullptr, need, "workspace"}});
    if (st != SCAN_OK) return st;
    RglruParams p{B, L, D, x, lx, la, alpha, reset, h0};
    LRS_TRY(launch_rglru_baseline(variant, p, (float*)workspace, y, y_dtype == SCAN_F32, h_final,
                                  (hipStream_t)stream),
            "rglru comparison scan");
    return SCAN_OK;
}

// --------------------------------------------- RG-LRU gate projections ---
static bool proj_shape(int B, int L, int D) {
    return B >= 1 && L >= 1 && (int64_t)B * L <= 0x7fffffff && D >= 256 && D <= 2560 && D % 256 == 0;
}

static void proj_bwd_layout(int BL, int D, float** dw_part, float** db_part, void* base, size_t* bytes) {
    Carver cv(base);
    const int nr = gate_proj_ranges(BL), Db = D / 16;
    float* a = cv.take<float>((size_t)nr * 2 * 16 * Db * Db);
    float* b = cv.take<float>((size_t)nr * 2 * D);
    if (dw_part) *dw_part = a;
    if (db_part) *db_part = b;
    if (bytes) *bytes = cv.off;
}

size_t rglru_gate_proj_bwd_workspace_bytes(int B, int L, int D) {
    if (!proj_shape(B, L, D)) return 0;
    size_t n = 0;
    proj_bwd_layout(B * L, D, nullptr, nullptr, nullptr, &n);
    return n;
}

scan_status rglru_gate_proj_fwd(int B, int L, int D, const void* x, const void* w_x, const float* b_x,
                                const void* w_a, const float* b_a, void* lx, void* la, void* stream) {
    if (!proj_shape(B, L, D))
        return fail(SCAN_ERR_SHAPE, "rglru_gate_proj_fwd: unsupported shape B=" + std::to_string(B) + " L=" +
                                        std::to_string(L) + " D=" + std::to_string(D) +
                                        " (need D a multiple of 256, 256 <= D <= 2560)");
    scan_status st = check_ptrs({{x, 0, "x"}, {w_x, 0, "w_x"}, {b_x, 0, "b_x"}, {w_a, 0, "w_a"}, {b_a, 0, "b_a"},
                                 {lx, 0, "lx"}, {la, 0, "la"}},
                                {});
    if (st != SCAN_OK) return st;
    const size_t BLD = (size_t)B * L * D, W = (size_t)D * (D / 16) * 2;
    st = check_alias({{x, BLD * 2, "x"}, {w_x, W, "w_x"}, {b_x, (size_t)D * 4, "b_x"}, {w_a, W, "w_a"},
                      {b_a, (size_t)D * 4, "b_a"}},
                     {{lx, BLD * 2, "lx"}, {la, BLD * 2, "la"}});
    if (st != SCAN_OK) return st;
    LRS_TRY(launch_gate_proj_fwd(B * L, D, x, w_x, b_x, w_a, b_a, lx, la, (hipStream_t)stream),
            "rglru gate projection");
    return SCAN_OK;
}

scan_status rglru_gate_proj_bwd(int B, int L, int D, const void* x, const void* w_x, const void* w_a,
                                const void* dlx, const void* dla, int grad_dtype, const void* dx_in, void* dx_out,
                                float* dw_x, float* db_x, float* dw_a, float* db_a, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!proj_shape(B, L, D))
        return fail(SCAN_ERR_SHAPE, "rglru_gate_proj_bwd: unsupported shape B=" + std::to_string(B) + " L=" +
                                        std::to_string(L) + " D=" + std::to_string(D));
    if (grad_dtype != SCAN_BF16 && grad_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "rglru_gate_proj_bwd: grad_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs({{x, 0, "x"}, {w_x, 0, "w_x"}, {w_a, 0, "w_a"}, {dlx, 0, "dlx"}, {dla, 0, "dla"},
                                 {dx_in, 0, "dx_in"}, {dx_out, 0, "dx_out"}, {dw_x, 0, "dw_x"}, {db_x, 0, "db_x"},
                                 {dw_a, 0, "dw_a"}, {db_a, 0, "db_a"}, {workspace, 0, "workspace"}},
                                {});
    if (st != SCAN_OK) return st;
    size_t need = 0;
    proj_bwd_layout(B * L, D, nullptr, nullptr, nullptr, &need);
    if (workspace_bytes < need)
        return fail(SCAN_ERR_WORKSPACE, "rglru_gate_proj_bwd: workspace_bytes " + std::to_string(workspace_bytes) +
                                            " < " + std::to_string(need));
    const size_t BLD = (size_t)B * L * D, W = (size_t)D * (D / 16) * 2, g = grad_dtype == SCAN_F32 ? 4 : 2;
    std::vector<Span> ins = {{x, BLD * 2, "x"}, {w_x, W, "w_x"}, {w_a, W, "w_a"}, {dlx, BLD * g, "dlx"},
                             {dla, BLD * g, "dla"}};
    // dx may be accumulated in place (dx_out == dx_in), never partly overlapped
    if (dx_in != dx_out) ins.push_back({dx_in, BLD * g, "dx_in"});
    st = check_alias(ins, {{dx_out, BLD * g, "dx_out"}, {dw_x, W * 2, "dw_x"}, {db_x, (size_t)D * 4, "db_x"},
                           {dw_a, W * 2, "dw_a"}, {db_a, (size_t)D * 4, "db_a"}, {workspace, need, "workspace"}});
    if (st != SCAN_OK) return st;
    float *dw_part, *db_part;
    proj_bwd_layout(B * L, D, &dw_part, &db_part, workspace, nullptr);
    LRS_TRY(launch_gate_proj_bwd(B * L, D, x, w_x, w_a, dlx, dla, grad_dtype == SCAN_F32, dx_in, dx_out, dw_x, db_x,
                                 dw_a, db_a, dw_part, db_part, (hipStream_t)stream),
            "rglru gate projection backward");
    return SCAN_OK;
}

// ------------------------------------------------------- SAMU decode ---
size_t samu_scan_decode_table_bytes(int D) {
    if (D < 8 || D % 8 != 0 || D > kMaxD) return 0;
    return samu_decode_table_floats(D / 2) * sizeof(float);
}

scan_status samu_scan_decode_prepare(int D, const float* w_phi, const float* w_r, const float* a_phi,
                                     const float* a_r, const float* nu, const float* theta, void* table,
                                     void* stream) {
    if (D < 8 || D % 8 != 0 || D > kMaxD)
        return fail(SCAN_ERR_SHAPE, "samu_scan_decode_prepare: unsupported D=" + std::to_string(D) +
                                        " (need 8 <= D <= 1048576 a multiple of 8)");
    scan_status st = check_ptrs({{w_phi, 0, "w_phi"}, {w_r, 0, "w_r"}, {a_phi, 0, "a_phi"}, {a_r, 0, "a_r"},
                                 {nu, 0, "nu"}, {theta, 0, "theta"}, {table, 0, "table"}},
                                {});
    if (st != SCAN_OK) return st;
    const int M = D / 2;
    st = check_alias({{w_phi, (size_t)(D + 1) * 4, "w_phi"}, {w_r, (size_t)(D + 1) * 4, "w_r"},
                      {a_phi, 4, "a_phi"}, {a_r, 4, "a_r"}, {nu, (size_t)M * 4, "nu"},
                      {theta, (size_t)M * 4, "theta"}},
                     {{table, samu_scan_decode_table_bytes(D), "table"}});
    if (st != SCAN_OK) return st;
    LRS_TRY(launch_samu_decode_prepare(D, w_phi, w_r, a_phi, a_r, nu, theta, (float*)table,
                                       (hipStream_t)stream),
            "samu decode table");
    return SCAN_OK;
}

scan_status samu_scan_decode(int B, int D, const void* x_sel, const void* b, const float* w_phi,
                             const float* w_r, const float* a_phi, const float* a_r, const float* nu,
                             const float* theta, const void* table, const float* z_in, float* z_out, void* y,
                             int y_dtype, void* stream) {
    if (B < 1 || B > 65535 || D < 8 || D % 8 != 0 || D > kMaxD)
        return fail(SCAN_ERR_SHAPE, "samu_scan_decode: unsupported shape B=" + std::to_string(B) +
                                        " D=" + std::to_string(D) +
                                        " (need 1 <= B <= 65535, 8 <= D <= 1048576 a multiple of 8)");
    if (y_dtype != SCAN_BF16 && y_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "samu_scan_decode: y_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs({{x_sel, 0, "x_sel"}, {b, 0, "b"}, {w_phi, 0, "w_phi"}, {w_r, 0, "w_r"},
                                 {a_phi, 0, "a_phi"}, {a_r, 0, "a_r"}, {nu, 0, "nu"}, {theta, 0, "theta"},
                                 {z_out, 0, "z_out"}, {y, 0, "y"}},
                                {{z_in, 0, "z_in"}, {table, 0, "table"}});
    if (st != SCAN_OK) return st;
    const int M = D / 2;
    const size_t BM = (size_t)B * M;
    std::vector<Span> ins = {{x_sel, (size_t)B * D * 2, "x_sel"}, {b, BM * 4, "b"},
                             {w_phi, (size_t)(D + 1) * 4, "w_phi"}, {w_r, (size_t)(D + 1) * 4, "w_r"},
                             {a_phi, 4, "a_phi"}, {a_r, 4, "a_r"}, {nu, (size_t)M * 4, "nu"},
                             {theta, (size_t)M * 4, "theta"},
                             {table, samu_scan_decode_table_bytes(D), "table"}};
    // the state may be updated in place (z_out == z_in), never partly overlapped
    if (z_in != z_out) ins.push_back({z_in, BM * 8, "z_in"});
    st = check_alias(ins, {{z_out, BM * 8, "z_out"}, {y, BM * 2 * (y_dtype == SCAN_F32 ? 4 : 2), "y"}});
    if (st != SCAN_OK) return st;
    LRS_TRY(launch_samu_decode(B, D, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, (const float*)table, z_in,
                               z_out, y, y_dtype == SCAN_F32, (hipStream_t)stream),
            "samu decode");
    return SCAN_OK;
}

// -------------------------------------------------------------- RG-LRU ---
size_t rglru_scan_saved_bytes(int B, int L, int D, int K) {
    Chunking ch;
    if (!rglru_shape(B, L, D, K, 0, &ch)) return 0;
    size_t n = 0;
    rg_saved_layout(nullptr, ch, D, &n);
    return n;
}

size_t rglru_scan_workspace_bytes(int B, int L, int D, int K, int G, int backward) {
    Chunking ch;
    if (!rglru_shape(B, L, D, K, G, &ch)) return 0;
    size_t n = 0;
    rg_ws_layout(nullptr, ch, D, backward != 0, &n);
    return n;
}

scan_status rglru_scan_fwd(int B, int L, int D, int K, int G, const void* x, const void* lx, const void* la,
                           const float* alpha, const unsigned char* reset, const float* h0, void* y,
                           int y_dtype, float* h_final, void* saved, void* workspace,
                           size_t workspace_bytes, void* stream) {
    Chunking ch;
    if (!rglru_shape(B, L, D, K, G, &ch))
        return fail(SCAN_ERR_SHAPE, "rglru_scan_fwd: unsupported shape " + shape_text(B, L, D, K, G) +
                                        " (need B, L >= 1, 2 <= D <= 1048576 even, K in {16, 32}, G >= 0,"
                                        " ceil(L/K) <= 65535)");
    if (y_dtype != SCAN_BF16 && y_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "rglru_scan_fwd: y_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs({{x, 0, "x"}, {lx, 0, "lx"}, {la, 0, "la"}, {alpha, 0, "alpha"}, {y, 0, "y"},
                                 {saved, 0, "saved"}, {workspace, 0, "workspace"}},
                                {{h0, 0, "h0"}, {h_final, 0, "h_final"}});
    if (st != SCAN_OK) return st;
    size_t need = 0, saved_n = 0;
    rg_ws_layout(nullptr, ch, D, false, &need);
    rg_saved_layout(nullptr, ch, D, &saved_n);
    if (workspace_bytes < need)
        return fail(SCAN_ERR_WORKSPACE, "rglru_scan_fwd: workspace_bytes " + std::to_string(workspace_bytes) +
                                            " < " + std::to_string(need));
    const size_t BL = (size_t)B * L, BLD = BL * D;
    st = check_alias({{x, BLD * 2, "x"}, {lx, BLD * 2, "lx"}, {la, BLD * 2, "la"}, {alpha, (size_t)D * 4, "alpha"},
                      {reset, BL, "reset"}, {h0, (size_t)B * D * 4, "h0"}},
                     {{y, BLD * (y_dtype == SCAN_F32 ? 4 : 2), "y"}, {h_final, (size_t)B * D * 4, "h_final"},
                      {saved, saved_n, "saved"}, {workspace, need, "workspace"}});
    if (st != SCAN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    RglruParams p{B, L, D, x, lx, la, alpha, reset, h0};
    RgSaved sv = rg_saved_layout(saved, ch, D, nullptr);
    RgWs ws = rg_ws_layout(workspace, ch, D, false, nullptr);
    if (rglru_fused(ch)) {
        LRS_TRY(launch_rglru_gscan(p, ch, ws.pub, ws.pub_bytes, sv.entries, y, y_dtype == SCAN_F32, h_final, s),
                "rglru forward scan");
        return SCAN_OK;
    }
    LRS_TRY(launch_rglru_summary(p, ch, ws.summ, s), "rglru chunk summary");
    LRS_TRY(launch_prefix(1, false, ch, D, PrefixSummaries{ws.summ, nullptr, nullptr, nullptr}, ws.gsum, h0,
                          sv.entries, s),
            "rglru prefix");
    LRS_TRY(launch_rglru_replay(p, ch, sv.entries, y, y_dtype == SCAN_F32, h_final, s), "rglru replay");
    return SCAN_OK;
}

scan_status rglru_scan_bwd(int B, int L, int D, int K, int G, const void* x, const void* lx, const void* la,
                           const float* alpha, const unsigned char* reset, const void* saved, const void* dy,
                           const float* dh_final, void* dx, void* dlx, void* dla, int grad_dtype,
                           float* dalpha, float* dh0, void* workspace, size_t workspace_bytes,
                           void* stream) {
    Chunking ch;
    if (!rglru_shape(B, L, D, K, G, &ch))
        return fail(SCAN_ERR_SHAPE, "rglru_scan_bwd: unsupported shape " + shape_text(B, L, D, K, G));
    if (grad_dtype != SCAN_BF16 && grad_dtype != SCAN_F32)
        return fail(SCAN_ERR_SHAPE, "rglru_scan_bwd: grad_dtype must be SCAN_BF16 or SCAN_F32");
    scan_status st = check_ptrs({{x, 0, "x"}, {lx, 0, "lx"}, {la, 0, "la"}, {alpha, 0, "alpha"},
                                 {saved, 0, "saved"}, {dy, 0, "dy"}, {dx, 0, "dx"}, {dlx, 0, "dlx"},
                                 {dla, 0, "dla"}, {dalpha, 0, "dalpha"}, {workspace, 0, "workspace"}},
                                {{dh_final, 0, "dh_final"}, {dh0, 0, "dh0"}});
    if (st != SCAN_OK) return st;
    size_t need = 0, saved_n = 0;
    rg_ws_layout(nullptr, ch, D, true, &need);
    rg_saved_layout(nullptr, ch, D, &saved_n);
    if (workspace_bytes < need)
        return fail(SCAN_ERR_WORKSPACE, "rglru_scan_bwd: workspace_bytes " + std::to_string(workspace_bytes) +
                                            " < " + std::to_string(need));
    const size_t BL = (size_t)B * L, BLD = BL * D;
    const size_t gsz = grad_dtype == SCAN_F32 ? 4 : 2;
    st = check_alias({{x, BLD * 2, "x"}, {lx, BLD * 2, "lx"}, {la, BLD * 2, "la"}, {alpha, (size_t)D * 4, "alpha"},
                      {reset, BL, "reset"}, {saved, saved_n, "saved"}, {dy, BLD * 2, "dy"},
                      {dh_final, (size_t)B * D * 4, "dh_final"}},
                     {{dx, BLD * gsz, "dx"}, {dlx, BLD * gsz, "dlx"}, {dla, BLD * gsz, "dla"},
                      {dalpha, (size_t)D * 4, "dalpha"}, {dh0, (size_t)B * D * 4, "dh0"},
                      {workspace, need, "workspace"}});
    if (st != SCAN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    RglruParams p{B, L, D, x, lx, la, alpha, reset, nullptr};
    RgSaved sv = rg_saved_layout(const_cast<void*>(saved), ch, D, nullptr);
    RgWs ws = rg_ws_layout(workspace, ch, D, true, nullptr);
    const int f32 = grad_dtype == SCAN_F32;
    if (rglru_fused(ch)) {
        LRS_TRY(launch_rglru_gbscan(p, ch, sv.entries, dh_final, ws.pub, ws.pub_bytes, dy, dx, dlx, dla, f32, dh0,
                                    ws.alpha_part, s),
                "rglru backward scan");
        LRS_TRY(launch_rglru_alpha_reduce(p, ws.alpha_rows, ws.alpha_part, dalpha, s), "rglru alpha reduction");
        return SCAN_OK;
    }
    LRS_TRY(launch_rglru_rev_summary(p, ch, dy, ws.summ, s), "rglru reverse summary");
    LRS_TRY(launch_prefix(1, true, ch, D, PrefixSummaries{ws.summ, nullptr, nullptr, nullptr}, ws.gsum,
                          dh_final, ws.carry, s),
            "rglru reverse prefix");
    LRS_TRY(launch_rglru_bwd_replay(p, ch, sv.entries, ws.carry, dy, dx, dlx, dla, f32, dh0, ws.alpha_part, s),
            "rglru backward replay");
    LRS_TRY(launch_rglru_alpha_reduce(p, ws.alpha_rows, ws.alpha_part, dalpha, s), "rglru alpha reduction");
    return SCAN_OK;
}

// ------------------------------------------------------------ profiler ---
int scan_set_handoff_poll_limit(int polls) {
    const int v = polls < 0 ? lrs::HANDOFF_POLLS_DEFAULT : polls;
    return lrs::g_handoff_polls.exchange(v);
}

void scan_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = on != 0;
}

int scan_profile_kernel_count(void) { return K_NUM_KERNELS; }

const char* scan_profile_kernel_name(int id) { return kernel_name(id); }

scan_status scan_profile_collect(double* total_ms, int* launches) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (total_ms) std::fill(total_ms, total_ms + K_NUM_KERNELS, 0.0);
    if (launches) std::fill(launches, launches + K_NUM_KERNELS, 0);
    scan_status st = SCAN_OK;
    for (const ProfRecord& r : g_prof_records) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == SCAN_OK) st = device_status(e, "scan_profile_collect");
        if (total_ms) total_ms[r.id] += ms;
        if (launches) launches[r.id] += 1;
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof_records.clear();
    return st;
}

}  // extern "C"
