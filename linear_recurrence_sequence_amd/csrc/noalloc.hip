// noalloc.hip -- samu_scan_fwd for callers that cannot allocate device memory
// (code under stream capture, tight serving loops): the forward workspace
// (the single-pass forward's hand-off words, or for groups longer than 16
// chunks the three-launch prefix's summaries and group states) lives in one
// file-scope device array instead of a caller buffer.
//
// Host code never passes the array's name to a kernel or a copy: on the host
// that name is only a stand-in for the symbol.  Its device address is looked
// up once per device, with that device current, and kept; the kernels receive
// that address exactly as they receive a caller's workspace.  Every call on a
// device shares that device's array, so calls that overlap in time on one
// device (two streams, or two host threads) race on it.  Nothing in the
// workspace has to start at zero: every word the forward kernels read was
// written earlier in the same call.
#include <mutex>
#include <string>

#include "internal.hpp"
#include "samu_scan.h"

namespace lrs {
namespace {

constexpr size_t kScratchBytes = SAMU_SCAN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on the first
// call made with the device current).
scan_status scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_last_error(SCAN_ERR_DEVICE, (std::string("samu_scan_fwd_noalloc: hipGetDevice: ") +
                                                                 hipGetErrorString(e)).c_str());
    if (dev < 0 || dev >= kMaxDevices)
        return set_last_error(SCAN_ERR_DEVICE, "samu_scan_fwd_noalloc: device index out of range");
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_last_error(SCAN_ERR_DEVICE, (std::string("samu_scan_fwd_noalloc: hipGetSymbolAddress: ") +
                                                     hipGetErrorString(e)).c_str());
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return SCAN_OK;
}

}  // namespace
}  // namespace lrs

extern "C" scan_status samu_scan_fwd_noalloc(int B, int L, int D, int K, int G, const void* x_sel, const void* b,
                                             const float* w_phi, const float* w_r, const float* a_phi,
                                             const float* a_r, const float* nu, const float* theta,
                                             const float* z0, void* y, int y_dtype, float* z_final, void* saved,
                                             void* stream) {
    const size_t need = samu_scan_workspace_bytes(B, L, D, K, G, 0);
    if (need == 0)  // unsupported shape: the forward's own check names the reason, before anything is enqueued
        return samu_scan_fwd(B, L, D, K, G, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0, y, y_dtype, z_final,
                             saved, nullptr, 0, stream);
    if (need > lrs::kScratchBytes)
        return lrs::set_last_error(SCAN_ERR_WORKSPACE,
                                   ("samu_scan_fwd_noalloc: the forward workspace of this shape (" +
                                    std::to_string(need) + " bytes) exceeds the static scratch of " +
                                    std::to_string(lrs::kScratchBytes) + " bytes; use samu_scan_fwd")
                                       .c_str());
    void* ws = nullptr;
    const scan_status st = lrs::scratch_ptr(&ws);
    if (st != SCAN_OK) return st;
    return samu_scan_fwd(B, L, D, K, G, x_sel, b, w_phi, w_r, a_phi, a_r, nu, theta, z0, y, y_dtype, z_final,
                         saved, ws, lrs::kScratchBytes, stream);
}
