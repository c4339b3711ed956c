// launch.hpp -- host entry points of the kernel translation units, called by
// the C ABI (api.hip) after argument validation.  Each function enqueues its
// launches on `s` and returns the first HIP error, if any.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace prn {

// Fill ranges of device memory with a 32- or 64-bit pattern in one launch
// (used instead of hipMemsetAsync so that every call stays a kernel-only
// sequence).
struct FillRange {
    void *ptr;
    uint64_t count;   // elements
    uint64_t value;   // pattern
    int bytes;        // 4 or 8
};
constexpr int kMaxFill = 8;

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Compute units of the current device (queried once per device).
int device_cu_count();
// Workgroups of `threads` threads of `kernel` that fit on one CU at once (at
// least 1).  Launchers keep the result in a function-local static, which C++
// initialises once and thread-safely.
int blocks_per_cu(const void *kernel, int threads);
hipError_t fill(const FillRange *r, int n, hipStream_t s);

hipError_t linscan_diag(int64_t B, int64_t L, int64_t H, const float *a, const float *b,
                        const float *h0, float *h, char *ws, hipStream_t s);
hipError_t linscan_blk2(int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                        const float *h0, float *h, char *ws, hipStream_t s);
// k x k blocks, k = 4 (hipErrorInvalidValue otherwise)
hipError_t linscan_blk(int k, int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                       const float *h0, float *h, char *ws, hipStream_t s);

struct GruFwdArgs {
    int64_t B, L, H;
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0;
    float *h;
    float tol;
    int32_t cap;
    int32_t *info;
    float *trace;
    int local;  // chained kernel: 1 workgroups own whole chains, 0 never, -1 choose
};
hipError_t gru_forward_step(const GruFwdArgs &a, char *ws, hipStream_t s);
hipError_t gru_forward_fused(const GruFwdArgs &a, hipStream_t s);
hipError_t gru_forward_chain(const GruFwdArgs &a, char *ws, hipStream_t s);

struct LstmFwdArgs {
    int64_t B, L, H;
    const float *pi, *pf, *po, *pg, *ui, *uf, *uo, *ug, *h0, *c0;
    float *h, *c;
    float tol;
    int32_t cap;
    int32_t *info;
    float *trace;
    int local;  // as for the GRU
};
hipError_t lstm_forward_step(const LstmFwdArgs &a, char *ws, hipStream_t s);
hipError_t lstm_forward_chain(const LstmFwdArgs &a, char *ws, hipStream_t s);

// Sequential application (one thread per channel; tol, cap, info, trace and
// local unused).
hipError_t gru_rollout(const GruFwdArgs &a, hipStream_t s);
hipError_t lstm_rollout(const LstmFwdArgs &a, hipStream_t s);

struct AdjArgs {
    int64_t B, L, H;
    const float *p[4], *u[4];
    const float *h0, *c0, *h, *c, *gh, *gc;
    float *gp[4], *gu[4];
    float *gh0, *gc0;
};
hipError_t gru_adjoint(const AdjArgs &a, char *ws, hipStream_t s);
hipError_t lstm_adjoint(const AdjArgs &a, char *ws, hipStream_t s);

size_t gru_adjoint_ws(int64_t B, int64_t L, int64_t H);
size_t lstm_adjoint_ws(int64_t B, int64_t L, int64_t H);

}  // namespace prn
