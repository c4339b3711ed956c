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

inline bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
inline bool aligned16(const void *p) { return aligned_to(p, 16); }

// The caller's workspace: its base (256-byte aligned) and its whole size in
// bytes (at the end of a tag period all of it but the header is cleared).
struct Ws {
    char *p;
    size_t bytes;
};

// Compute units of the current device (queried once per device).
int device_cu_count();
// Workgroups of `threads` threads of `kernel` that fit on one CU at once (at
// least 1).  Launchers keep the result in a function-local static, which C++
// initialises once and thread-safely.
int blocks_per_cu(const void *kernel, int threads);
hipError_t fill(const FillRange *r, int n, hipStream_t s);

hipError_t linscan_diag(int64_t B, int64_t L, int64_t H, const float *a, const float *b,
                        const float *h0, float *h, const Ws &ws, hipStream_t s);
hipError_t linscan_blk2(int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                        const float *h0, float *h, const Ws &ws, hipStream_t s);
// k x k blocks, k = 4 (hipErrorInvalidValue otherwise)
hipError_t linscan_blk(int k, int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                       const float *h0, float *h, const Ws &ws, hipStream_t s);

// k x k blocks with each block's rows on a lane group, k = 4 or 8
// (hipErrorInvalidValue otherwise); workspace blkrow_ws
hipError_t linscan_blkrow(int k, int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                          const float *h0, float *h, const Ws &ws, hipStream_t s);
// Newton forward of the GRU with dense recurrence inside heads of k
// channels (k = 4, 8): tensors [B, L, NH, k], U [NH, k, k].
struct HgruFwdArgs {
    int k;
    int64_t B, L, NH;
    const float *pz, *pr, *pc, *Uz, *Ur, *Uc, *h0, *h_init;
    float *h;
    float tol;
    int32_t cap;
    int32_t *info;
    float *trace;
};
hipError_t hgru_forward(const HgruFwdArgs &a, const Ws &ws, hipStream_t s);
struct HgruBwdArgs {
    int k;
    int64_t B, L, NH;
    const float *pz, *pr, *pc, *Uz, *Ur, *Uc, *h0, *h, *gh;
    float *gpz, *gpr, *gpc;
    float *gU[3];  // dL/dUz, dL/dUr, dL/dUc [NH, k, k], each or null
    float *gh0;
};
hipError_t hgru_backward(const HgruBwdArgs &a, const Ws &ws, hipStream_t s);
struct GruFwdArgs {
    int64_t B, L, H;
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0;
    const float *h_init;  // Newton's initial iterate [B, L, H], or null for zeros
    float *h;
    float tol;
    int32_t cap;
    int32_t *info;
    float *trace;
    int local;  // chained kernel: 1 workgroups own whole chains, 0 never, -1 choose
};
hipError_t gru_forward_step(const GruFwdArgs &a, const Ws &ws, hipStream_t s);
hipError_t gru_forward_fused(const GruFwdArgs &a, hipStream_t s);
hipError_t gru_forward_chain(const GruFwdArgs &a, const Ws &ws, hipStream_t s);

struct LstmFwdArgs {
    int64_t B, L, H;
    const float *pi, *pf, *po, *pg, *ui, *uf, *uo, *ug, *h0, *c0;
    const float *h_init, *c_init;  // initial iterates [B, L, H]; a null one is zero
    float *h, *c;
    float tol;
    int32_t cap;
    int32_t *info;
    float *trace;
    int local;  // as for the GRU
};
hipError_t lstm_forward_step(const LstmFwdArgs &a, const Ws &ws, hipStream_t s);
hipError_t lstm_forward_chain(const LstmFwdArgs &a, const Ws &ws, hipStream_t s);

// Whether the chained Newton forward at this shape lets each workgroup own
// whole chains of chunks (no workspace beyond the header) rather than
// chaining chunks across workgroups; local as in GruFwdArgs.
bool gru_chain_owns_chains(int64_t B, int64_t L, int64_t H, int local);
bool lstm_chain_owns_chains(int64_t B, int64_t L, int64_t H, int local);

// Sequential application (one thread per channel; tol, cap, info, trace and
// local unused).
hipError_t gru_rollout(const GruFwdArgs &a, hipStream_t s);
hipError_t lstm_rollout(const LstmFwdArgs &a, hipStream_t s);

// info = {first k with max|delta| <= tol, 1} or {cap, 0}, trace[k-1] =
// max|delta| of iteration k, from the per-iteration slots of a workspace
// (either output may be null).
hipError_t newton_finalize_launch(const uint32_t *maxd, int cap, float tol, int32_t *info, float *trace,
                                  hipStream_t s);
// Warm start of a per-iteration path on a one-component state of H
// channels per batch row and chunks of T positions: init copied into h, and
// its state at the last position of every chunk into bnd [chunk][B][H].
hipError_t newton_seed1(const float *init, float *h, float *bnd, int64_t B, int64_t L, int64_t H, int64_t T,
                        hipStream_t s);
struct AdjArgs {
    int64_t B, L, H;
    const float *p[4], *u[4];
    const float *h0, *c0, *h, *c, *gh, *gc;
    float *gp[4], *gu[4];
    float *gh0, *gc0;
};
hipError_t gru_adjoint(const AdjArgs &a, const Ws &ws, hipStream_t s);
hipError_t lstm_adjoint(const AdjArgs &a, const Ws &ws, hipStream_t s);

size_t gru_adjoint_ws(int64_t B, int64_t L, int64_t H);
size_t lstm_adjoint_ws(int64_t B, int64_t L, int64_t H);

}  // namespace prn
