// rollout.hip -- sequential application of the cells: one thread per channel
// walks the sequence in order, one cell evaluation per position.  This is the
// evaluation the pages measure their speedups against (ParaRNN page, abstract
// and Fig. 2 caption: speedup over sequential application; DEER summary page,
// results paragraph: sequential evaluation of a GRU at L = 2^20).  It is exact
// (no iteration) and does one cell per element where Newton does one per
// element and iteration, but it can only use B*H threads.
//
// Thread n is channel (b, j) = (n / H, n % H), so a wave's loads and stores
// at one position are consecutive channels of one row (coalesced once
// H >= 64).  The gate inputs of the next U positions are loaded while the
// current U are evaluated (two register sets), so U positions of every gate
// are in flight per thread.
#include "cells.hpp"
#include "launch.hpp"

namespace prn {

namespace {
constexpr int kRollThreads = 64;  // one wave per workgroup: small B*H still spreads over the CUs
constexpr int kRollU = 16;        // positions per block of loads
}

template <int NG>
struct RollBlock {
    float x[NG][kRollU];
};

template <int NG>
__device__ __forceinline__ void roll_load(const float *const (&p)[NG], int64_t base, int64_t t0, int64_t L,
                                          int64_t H, RollBlock<NG> &blk) {
#pragma unroll
    for (int i = 0; i < kRollU; ++i) {
        const bool v = t0 + i < L;
        const int64_t o = base + (v ? (t0 + i) * H : 0);
#pragma unroll
        for (int g = 0; g < NG; ++g) blk.x[g][i] = v ? ld_once(p[g] + o) : 0.0f;
    }
}

__global__ __launch_bounds__(kRollThreads) void gru_rollout_kernel(GruFwdArgs a) {
    const int64_t n = (int64_t)blockIdx.x * kRollThreads + threadIdx.x;
    if (n >= a.B * a.H) return;
    const int64_t b = n / a.H, j = n - b * a.H;
    const int64_t base = b * a.L * a.H + j;
    const float uz = a.uz[j], ur = a.ur[j], uc = a.uc[j];
    const float *const p[3] = {a.pz, a.pr, a.pc};
    float h = a.h0 != nullptr ? a.h0[n] : 0.0f;
    RollBlock<3> cur, nxt{};
    roll_load<3>(p, base, 0, a.L, a.H, cur);
    for (int64_t t0 = 0; t0 < a.L; t0 += kRollU) {
        if (t0 + kRollU < a.L) roll_load<3>(p, base, t0 + kRollU, a.L, a.H, nxt);
#pragma unroll
        for (int i = 0; i < kRollU; ++i) {
            if (t0 + i < a.L) {
                float F, J;
                gru_f_j(h, cur.x[0][i], cur.x[1][i], cur.x[2][i], uz, ur, uc, F, J);
                h = F;
                a.h[base + (t0 + i) * a.H] = h;
            }
        }
        cur = nxt;
    }
}

__global__ __launch_bounds__(kRollThreads) void lstm_rollout_kernel(LstmFwdArgs a) {
    const int64_t n = (int64_t)blockIdx.x * kRollThreads + threadIdx.x;
    if (n >= a.B * a.H) return;
    const int64_t b = n / a.H, j = n - b * a.H;
    const int64_t base = b * a.L * a.H + j;
    const float ui = a.ui[j], uf = a.uf[j], uo = a.uo[j], ug = a.ug[j];
    const float *const p[4] = {a.pi, a.pf, a.po, a.pg};
    float h = a.h0 != nullptr ? a.h0[n] : 0.0f;
    float c = a.c0 != nullptr ? a.c0[n] : 0.0f;
    RollBlock<4> cur, nxt{};
    roll_load<4>(p, base, 0, a.L, a.H, cur);
    for (int64_t t0 = 0; t0 < a.L; t0 += kRollU) {
        if (t0 + kRollU < a.L) roll_load<4>(p, base, t0 + kRollU, a.L, a.H, nxt);
#pragma unroll
        for (int i = 0; i < kRollU; ++i) {
            if (t0 + i < a.L) {
                const Lstm2 r = lstm_f_j(c, h, cur.x[0][i], cur.x[1][i], cur.x[2][i], cur.x[3][i], ui, uf, uo, ug);
                c = r.Fc;
                h = r.Fh;
                const int64_t o = base + (t0 + i) * a.H;
                a.c[o] = c;
                a.h[o] = h;
            }
        }
        cur = nxt;
    }
}

hipError_t gru_rollout(const GruFwdArgs &a, hipStream_t s) {
    const int64_t grid = (a.B * a.H + kRollThreads - 1) / kRollThreads;
    hipLaunchKernelGGL(gru_rollout_kernel, dim3((unsigned)grid), dim3(kRollThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t lstm_rollout(const LstmFwdArgs &a, hipStream_t s) {
    const int64_t grid = (a.B * a.H + kRollThreads - 1) / kRollThreads;
    hipLaunchKernelGGL(lstm_rollout_kernel, dim3((unsigned)grid), dim3(kRollThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace prn
