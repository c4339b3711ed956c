// noalloc.hip -- pararnn_gru_forward_noalloc: the GRU Newton forward with
// its workspace taken from a static device array of the library instead of
// the caller, for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives once per device for the life of the process.  Its device
// address is obtained once per device, with that device current, by
// hipGetSymbolAddress; the first call on a device also zero-fills the array
// with the library's fill kernel on the caller's stream (the workspace rules
// of every entry point: zero-filled before first use, kept valid by each
// call afterwards).  From then on the array is an ordinary workspace: every
// call on a device shares it and finds the last call's contents, which the
// launch tags make harmless.  Calls that overlap in time on one device (on
// different streams or threads) race on it and must not be issued.
#include <mutex>

#include "pararnn.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)PARARNN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_setup;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, guarded by g_setup

// Device address of the array on the current device, set up on first use.
int scratch_address(void **out, hipStream_t s) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PARARNN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_setup);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PARARNN_ERR_HIP;
        prn::FillRange fr[1] = {{p, kScratchBytes / 8, 0, 8}};
        if (prn::fill(fr, 1, s) != hipSuccess) return PARARNN_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PARARNN_OK;
}

}  // namespace

extern "C" int pararnn_gru_forward_noalloc(int64_t B, int64_t L, int64_t H, const float *pz, const float *pr,
                                           const float *pc, const float *uz, const float *ur, const float *uc,
                                           const float *h0, float *h, float tol, int32_t max_iter, int32_t *info,
                                           float *trace, void *stream) {
    const size_t need = pararnn_workspace_bytes(PARARNN_OP_GRU_FORWARD, B, L, H, max_iter);
    if (need == 0) return PARARNN_ERR_INVALID;
    if (need > kScratchBytes) return PARARNN_ERR_TOO_LARGE;
    void *ws = nullptr;
    const int st = scratch_address(&ws, static_cast<hipStream_t>(stream));
    if (st != PARARNN_OK) return st;
    return pararnn_gru_forward(B, L, H, pz, pr, pc, uz, ur, uc, h0, nullptr, h, tol, max_iter, info, trace, ws,
                               kScratchBytes, stream);
}
