// gru_fused.hip -- the whole Newton routine for the GRU-style cell in one
// kernel, with the sequence kept on chip between iterations (ParaRNN page,
// Fig. 2 right and Fig. 5: the fully fused solver is the fastest modality).
//
// One workgroup (8 waves) owns all L <= 32*C positions of 16 channels of one
// batch row.  Lane l of wave w handles channel (l mod 16) and sub-chunk
// 4w + l/16 of C consecutive positions.  The gate inputs are read from HBM
// once, the iterate, the Jacobians and the residuals live in registers, and
// h is written once.  Per iteration:
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
constexpr int kCh = kFusedChannels;       // channels per workgroup
constexpr int kSubW = 64 / kCh;           // sub-chunks per wave
constexpr int kNW = kFusedSubchunks / kSubW;  // waves per workgroup
static_assert(kCh * kSubW == 64, "a wave is kCh channels x kSubW sub-chunks");
}  // namespace

struct FusedGruArgs {
    int64_t B, L, H, ncb;
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0;
    float *h;
    float tol;
    int32_t cap;
    int32_t *info;
    uint32_t *trace;
};

template <int C>
__global__ __launch_bounds__(kNW * 64) void gru_fused_kernel(FusedGruArgs a) {
    __shared__ Aff1 s_wtot[kNW][kCh];
    __shared__ float s_last[kFusedSubchunks][kCh];
    __shared__ uint32_t s_wmax[kNW];

    // XCD-aware tile order: workgroups are dispatched round-robin over the 8
    // XCDs, so give each XCD a contiguous run of tiles; neighbouring
    // 16-channel tiles share 128-byte lines and then share one L2.
    const int64_t nblk = gridDim.x;
    int64_t tile = blockIdx.x;
    if ((nblk & 7) == 0) tile = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int64_t b = tile / a.ncb;
    const int64_t cb = tile - b * a.ncb;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane % kCh, sl = lane / kCh;
    const int sub = w * kSubW + sl;
    const int64_t j = cb * kCh + ch;
    const bool ok = j < a.H;
    const int64_t t0 = (int64_t)sub * C;
    const int64_t L = a.L, H = a.H;
    const int64_t base = (b * L + t0) * H + j;

    float xz[C], xr[C], xc[C], hv[C], Jv[C], bv[C];
    bool val[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        val[i] = ok && (t0 + i < L);
        xz[i] = val[i] ? a.pz[base + i * H] : 0.0f;
        xr[i] = val[i] ? a.pr[base + i * H] : 0.0f;
        xc[i] = val[i] ? a.pc[base + i * H] : 0.0f;
        hv[i] = 0.0f;
    }
    const float wz = ok ? a.uz[j] : 0.0f, wr = ok ? a.ur[j] : 0.0f, wc = ok ? a.uc[j] : 0.0f;
    const float hinit = (ok && a.h0 != nullptr) ? a.h0[b * H + j] : 0.0f;

    int iters = 0;
    bool conv = false;
    for (int k = 1; k <= a.cap; ++k) {
        float hp = 0.0f;
        if (sub == 0)
            hp = hinit;
        else if (k > 1)
            hp = s_last[sub - 1][ch];

        Aff1 acc = {1.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float F, J;
            gru_f_j(hp, xz[i], xr[i], xc[i], wz, wr, wc, F, J);
            Jv[i] = val[i] ? J : 1.0f;
            bv[i] = val[i] ? F - hv[i] : 0.0f;
            hp = hv[i];
            acc = {acc.a * Jv[i], fmaf(Jv[i], acc.b, bv[i])};
        }

        // scan of the sub-chunk maps of each channel
        Aff1 incl = acc;
#pragma unroll
        for (int d = 1; d < kSubW; d <<= 1) {
            const Aff1 o = MonoidT<1>::shfl_up(incl, d * kCh);
            if (sl >= d) incl = MonoidT<1>::then(o, incl);
        }
        Aff1 exw = MonoidT<1>::shfl_up(incl, kCh);
        if (sl == 0) exw = MonoidT<1>::id();
        if (sl == kSubW - 1) s_wtot[w][ch] = incl;
        __syncthreads();
        Aff1 pre = MonoidT<1>::id();
        for (int ww = 0; ww < w; ++ww) pre = MonoidT<1>::then(pre, s_wtot[ww][ch]);
        float d = MonoidT<1>::then(pre, exw).b;  // delta entering the sub-chunk (delta_{-1} = 0)

        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            d = fmaf(Jv[i], d, bv[i]);
            hv[i] += d;
            const uint32_t ad = val[i] ? abs_bits(d) : 0u;
            mx = ad > mx ? ad : mx;
        }
        s_last[sub][ch] = hv[C - 1];
        mx = wave_max_u32(clamp_nan_to_inf(mx));
        if (lane == 0) s_wmax[w] = mx;
        __syncthreads();
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < kNW; ++ww) m = s_wmax[ww] > m ? s_wmax[ww] : m;
        iters = k;
        if (threadIdx.x == 0 && a.trace != nullptr)
            __hip_atomic_fetch_max(a.trace + (k - 1), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__uint_as_float(m) <= a.tol) {
            conv = true;
            break;
        }
    }

#pragma unroll
    for (int i = 0; i < C; ++i)
        if (val[i]) a.h[base + i * H] = hv[i];
    if (threadIdx.x == 0 && a.info != nullptr) {
        __hip_atomic_fetch_max(a.info, iters, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!conv) __hip_atomic_fetch_and(a.info + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int C>
static hipError_t launch_fused(const FusedGruArgs &fa, int64_t nblocks, hipStream_t s) {
    hipLaunchKernelGGL(gru_fused_kernel<C>, dim3((unsigned)nblocks), dim3(kNW * 64), 0, s, fa);
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
    fa.h = a.h;
    fa.tol = a.tol;
    fa.cap = a.cap;
    fa.info = a.info;
    fa.trace = reinterpret_cast<uint32_t *>(a.trace);
    FillRange fr[3] = {
        {a.info, a.info ? 1ull : 0ull, 0, 4},                                // iterations = 0
        {a.info ? a.info + 1 : nullptr, a.info ? 1ull : 0ull, 1, 4},         // converged = 1
        {a.trace, a.trace ? (uint64_t)a.cap : 0ull, 0, 4},
    };
    hipError_t e = fill(fr, 3, s);
    if (e != hipSuccess) return e;
    const int64_t nblocks = a.B * fa.ncb;
    switch (C) {
        case 1: return launch_fused<1>(fa, nblocks, s);
        case 2: return launch_fused<2>(fa, nblocks, s);
        case 4: return launch_fused<4>(fa, nblocks, s);
        case 8: return launch_fused<8>(fa, nblocks, s);
        case 16: return launch_fused<16>(fa, nblocks, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace prn
