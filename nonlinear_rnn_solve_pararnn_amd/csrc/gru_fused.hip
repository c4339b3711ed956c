// gru_fused.hip -- the whole Newton routine for the GRU-style cell in one
// kernel, with the sequence kept on chip between iterations (ParaRNN page,
// Fig. 2 right and Fig. 5: the fully fused solver is the fastest modality).
//
// A tile is all L <= 32*C positions of 16 channels of one batch row, owned by
// one workgroup of 8 waves: lane l of wave w handles channel (l mod 16) and
// sub-chunk 4w + l/16 of C consecutive positions.  The gate inputs are read
// from HBM once, the iterate, the Jacobians and the residuals live in
// registers, and h is written once.  Per iteration:
//   1. every thread evaluates its C cells at the previous iterate (the state
//      before its first position comes from the neighbouring sub-chunk
//      through LDS) and composes its sub-chunk's affine map
//      delta -> J delta + beta with beta = F - h;
//   2. the 32 sub-chunk maps of each channel are scanned: two shuffle steps
//      across the 4 lane groups of a wave, then across the 8 waves in LDS;
//   3. every thread applies its carry-in delta, updates h += delta and
//      forms max|delta|; the workgroup maximum decides convergence of this
//      tile (each tile stops on its own once its max|delta| <= tol).

#include "cells.hpp"
#include "launch.hpp"

namespace prn {

namespace {
constexpr int kCh = kFusedChannels;           // channels per tile
constexpr int kSubW = 64 / kCh;               // sub-chunks per wave
constexpr int kNW = kFusedSubchunks / kSubW;  // waves per workgroup
static_assert(kCh * kSubW == 64, "a wave is kCh channels x kSubW sub-chunks");
constexpr float kE1 = -kLog2e, kE2 = -2.0f * kLog2e;
}  // namespace

struct FusedGruArgs {
    int64_t B, L, H, ncb;
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0;
    const float *h_init;  // initial iterate [B, L, H], or null for zeros
    float *h;
    float tol;
    int32_t cap;
    int32_t *info;
    uint32_t *trace;
};

// XCD-aware tile order: workgroups are dispatched round-robin over the 8 XCDs,
// so give each XCD a contiguous run of tiles; neighbouring 16-channel tiles
// share 128-byte lines and then share one L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t n, int64_t ntiles) {
    if (!kFusedXcdOrder) return n;
    return (ntiles & 7) == 0 ? (n & 7) * (ntiles >> 3) + (n >> 3) : n;
}

// Newton iterations on one tile held in registers.  x* are the pre-scaled
// gate inputs (pz, pr by -log2 e; pc by -2 log2 e); hv holds the initial
// iterate when `warm` (zero otherwise) and receives the solution.
//
// Arithmetic per position and iteration (h the previous state, hc the current
// one): each gate is one fma, one exp2, one add and one reciprocal; then
//   c = 2 s - 1, F = h + z (c - h),
//   J = (1-z) + z [ (1-z) uz (c-h) + (1-c^2) uc (r + h r(1-r) ur) ],
//   beta = F - hc.
// |delta| is tracked with a float max (which ignores NaN); a NaN anywhere in a
// thread's chain propagates to its last delta, which is checked once.
template <int C, int NSUB, int CH, bool FULL>
__device__ __forceinline__ void newton_on_tile(const float (&xz)[C], const float (&xr)[C],
                                               const float (&xc)[C], float (&hv)[C],
                                               const bool (&val)[C], bool ok, float uz, float ur,
                                               float uc, float hinit, bool warm, const FusedGruArgs &a,
                                               int &iters, bool &conv) {
    constexpr int SUBW = 64 / CH;     // sub-chunks per wave
    constexpr int NW = NSUB / SUBW;   // waves of the workgroup
    __shared__ Aff1 s_wtot[NW][CH];
    __shared__ float s_last[NSUB][CH];
    __shared__ float s_wmax[NW];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane % CH, sl = lane / CH;
    const int sub = w * SUBW + sl;
    const GruScaledW gw = gru_scaled_weights(uz, ur, uc);
    float Jv[C], bv[C];
    if (warm) {
        // the initial iterate's last state of every sub-chunk, for its successor
        s_last[sub][ch] = hv[C - 1];
        lds_barrier();
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) hv[i] = 0.0f;
    }
    iters = 0;
    conv = false;
    for (int k = 1; k <= a.cap; ++k) {
        float hp = 0.0f;
        if (sub == 0)
            hp = hinit;
        else if (k > 1 || warm)
            hp = s_last[sub - 1][ch];

        Aff1 acc = {1.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float J, beta;
            gru_map_scaled(gw, hp, xz[i], xr[i], xc[i], hv[i], J, beta);
            if (!FULL) {
                J = val[i] ? J : 1.0f;
                beta = val[i] ? beta : 0.0f;
            }
            Jv[i] = J;
            bv[i] = beta;
            hp = hv[i];
            acc = {acc.a * J, fmaf(J, acc.b, beta)};
        }

        // scan of the sub-chunk maps of each channel
        Aff1 incl = acc;
#pragma unroll
        for (int d = 1; d < SUBW; d <<= 1) {
            const Aff1 o = MonoidT<1>::shfl_up(incl, d * CH);
            if (sl >= d) incl = MonoidT<1>::then(o, incl);
        }
        Aff1 exw = MonoidT<1>::shfl_up(incl, CH);
        if (sl == 0) exw = MonoidT<1>::id();
        if (sl == SUBW - 1) s_wtot[w][ch] = incl;
        lds_barrier();
        Aff1 pre = MonoidT<1>::id();
        for (int ww = 0; ww < w; ++ww) pre = MonoidT<1>::then(pre, s_wtot[ww][ch]);
        float d = MonoidT<1>::then(pre, exw).b;  // delta entering the sub-chunk (delta_{-1} = 0)

        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            d = fmaf(Jv[i], d, bv[i]);
            hv[i] += d;
            mx = fmaxf(mx, fabsf(d));
        }
        if (d != d) mx = __uint_as_float(kInfBits);
        if (!ok) mx = 0.0f;
        s_last[sub][ch] = hv[C - 1];
        mx = __uint_as_float(wave_max_u32(__float_as_uint(mx)));
        if (lane == 0) s_wmax[w] = mx;
        lds_barrier();
        float m = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, s_wmax[ww]);
        iters = k;
        if (threadIdx.x == 0 && a.trace != nullptr) {
            // shared by every workgroup: skip the atomic unless it would raise the value
            const uint32_t cur = __hip_atomic_load(a.trace + (k - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__float_as_uint(m) > cur)
                __hip_atomic_fetch_max(a.trace + (k - 1), __float_as_uint(m), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        if (m <= a.tol) {
            conv = true;
            break;
        }
    }
    // s_last and s_wmax are rewritten by the next tile's first iteration
    lds_barrier();
}

__device__ __forceinline__ void report_tile(const FusedGruArgs &a, int iters, bool conv) {
    if (threadIdx.x == 0 && a.info != nullptr) {
        // shared by every workgroup: skip atomics that would not change the value
        if (iters > __hip_atomic_load(a.info, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            __hip_atomic_fetch_max(a.info, iters, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!conv && __hip_atomic_load(a.info + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
            __hip_atomic_store(a.info + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One tile per workgroup.  FULL: every lane's channel exists and every
// position is inside the sequence (L == 32*C, H a multiple of 16).
template <int C, bool FULL>
__global__ __launch_bounds__(kNW * 64, 4) void gru_fused_kernel(FusedGruArgs a) {
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t b = tile / a.ncb;
    const int64_t cb = tile - b * a.ncb;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane % kCh, sl = lane / kCh;
    const int sub = w * kSubW + sl;
    const int64_t j = cb * kCh + ch;
    const bool ok = FULL || j < a.H;
    const int64_t t0 = (int64_t)sub * C;
    const int64_t L = a.L, H = a.H;
    const int64_t base = (b * L + t0) * H + j;

    float xz[C], xr[C], xc[C], hv[C];
    bool val[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        // every load issued, none behind a branch (a position outside reads
        // element 0), so they are all in flight together; scaled afterwards
        val[i] = FULL || (ok && (t0 + i < L));
        const int64_t e = val[i] ? base + i * H : 0;
        xz[i] = a.pz[e];
        xr[i] = a.pr[e];
        xc[i] = a.pc[e];
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {
        xz[i] = val[i] ? kE1 * xz[i] : 0.0f;
        xr[i] = val[i] ? kE1 * xr[i] : 0.0f;
        xc[i] = val[i] ? kE2 * xc[i] : 0.0f;
    }
    const float uz = ok ? a.uz[j] : 0.0f, ur = ok ? a.ur[j] : 0.0f, uc = ok ? a.uc[j] : 0.0f;
    const float hinit = (ok && a.h0 != nullptr) ? a.h0[b * H + j] : 0.0f;
    const bool warm = a.h_init != nullptr;
    if (warm) {
#pragma unroll
        for (int i = 0; i < C; ++i) hv[i] = val[i] ? a.h_init[base + i * H] : 0.0f;
    }
    int iters;
    bool conv;
    newton_on_tile<C, kFusedSubchunks, kCh, FULL>(xz, xr, xc, hv, val, ok, uz, ur, uc, hinit, warm, a, iters,
                                                  conv);
#pragma unroll
    for (int i = 0; i < C; ++i)
        if (val[i]) a.h[base + i * H] = hv[i];
    report_tile(a, iters, conv);
}

template <int C>
static hipError_t launch_fused(const FusedGruArgs &fa, int64_t ntiles, hipStream_t s) {
    const bool full = fa.L == (int64_t)kFusedSubchunks * C && fa.H % kCh == 0;
    if (full)
        hipLaunchKernelGGL((gru_fused_kernel<C, true>), dim3((unsigned)ntiles), dim3(kNW * 64), 0, s, fa);
    else
        hipLaunchKernelGGL((gru_fused_kernel<C, false>), dim3((unsigned)ntiles), dim3(kNW * 64), 0, s, fa);
    return hipGetLastError();
}

hipError_t gru_forward_fused(const GruFwdArgs &a, hipStream_t s) {
    const int C = fused_c_for(a.L);
    if (C == 0) return hipErrorInvalidValue;
    FusedGruArgs fa;
    fa.B = a.B;
    fa.L = a.L;
    fa.H = a.H;
    fa.ncb = (a.H + kCh - 1) / kCh;
    fa.pz = a.pz;
    fa.pr = a.pr;
    fa.pc = a.pc;
    fa.uz = a.uz;
    fa.ur = a.ur;
    fa.uc = a.uc;
    fa.h0 = a.h0;
    fa.h_init = a.h_init;
    fa.h = a.h;
    fa.tol = a.tol;
    fa.cap = a.cap;
    fa.info = a.info;
    fa.trace = reinterpret_cast<uint32_t *>(a.trace);
    FillRange fr[3] = {
        {a.info, a.info ? 1ull : 0ull, 0, 4},                         // iterations = 0
        {a.info ? a.info + 1 : nullptr, a.info ? 1ull : 0ull, 1, 4},  // converged = 1
        {a.trace, a.trace ? (uint64_t)a.cap : 0ull, 0, 4},
    };
    hipError_t e = fill(fr, 3, s);
    if (e != hipSuccess) return e;
    const int64_t ntiles = a.B * fa.ncb;
    switch (C) {
        case 1: return launch_fused<1>(fa, ntiles, s);
        case 2: return launch_fused<2>(fa, ntiles, s);
        case 4: return launch_fused<4>(fa, ntiles, s);
        case 8: return launch_fused<8>(fa, ntiles, s);
        case 16: return launch_fused<16>(fa, ntiles, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace prn
