// scan_core.hpp -- single-pass chunked scan of a linear recurrence over the
// sequence axis, the solver of the bi-diagonal systems that Newton's method
// produces (ParaRNN page, TL;DR and Fig. 2: parallel reduction of the block
// bi-diagonal system; DEER summary: associative scan).
//
// Work decomposition (four levels, all composing the affine maps of
// common.hpp):
//   1. each thread runs serially over C consecutive positions of one channel
//      and forms the aggregate map of that sub-chunk;
//   2. the workgroup combines its sub-chunks: across waves through LDS when
//      the 64 lanes of a wave are 64 channels ("channel lanes", for H >= 32;
//      every global access is then a coalesced 256-byte row segment), or by a
//      shuffle scan across the lanes plus LDS across waves when all threads
//      of the workgroup walk one channel ("time lanes", for small H such as
//      H = 1);
//   3. workgroups along the sequence axis are chained by a decoupled
//      look-back (common.hpp) in the order of dynamically drawn tickets;
//   4. each thread applies its carry-in and re-runs its C positions, which
//      are still in registers, so inputs are read from HBM exactly once.
//
// The per-position arithmetic comes from an Op (linear scan, one Newton
// iteration of a cell, or the adjoint of a cell): phase1 loads a sub-chunk
// and returns its aggregate map; phase2 receives the state entering the
// sub-chunk, finishes it and stores results.
#pragma once

#include "common.hpp"

namespace prn {

struct ScanGeo {
    int64_t B, L, H;
    int64_t ncb;            // channel blocks per batch row (channel lanes: ceil(H/64); time lanes: H)
    int64_t nq;             // chunks along the sequence
    uint32_t *counter;      // ticket counter, zero at launch
    uint64_t *agg, *inc;    // look-back descriptors [nq][B][H] (words per descriptor: Desc<S>)
    uint64_t *agg_next, *inc_next;  // optional: descriptor set to reset for the next launch
    uint32_t *err;          // optional: set to 1 if a look-back wait gave up
};

struct TilePos {
    int64_t tile;           // workgroup ticket: (q * B + b) * ncb + channel block
    int64_t b, j, q, pos0;  // batch row, channel, chunk index, first position of this thread
    int sub, nsub;          // sub-chunk index of this thread within the chunk, and count
    bool ok;                // channel exists (j < H)
};

template <class Op, int NW, int C, bool CHANNEL_LANES>
__global__ __launch_bounds__(NW * 64) void chunk_scan_kernel(Op op, ScanGeo g) {
    constexpr int S = Op::S;
    using M = MonoidT<S>;
    using D = Desc<S>;
    using Map = typename M::Map;
    using State = typename M::State;
    constexpr int NT = NW * 64;
    constexpr int64_t T = CHANNEL_LANES ? (int64_t)NW * C : (int64_t)NT * C;

    __shared__ Map s_part[CHANNEL_LANES ? NT : NW];
    __shared__ State s_carry[CHANNEL_LANES ? 64 : 1];
    __shared__ uint32_t s_ticket;

    if (!op.active()) return;  // uniform over the grid (e.g. Newton already converged)

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0)
        s_ticket = __hip_atomic_fetch_add(g.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t ticket = s_ticket;
    const int64_t per_q = g.B * g.ncb;

    TilePos tp;
    tp.tile = ticket;
    tp.q = ticket / per_q;
    const int64_t rest = ticket - tp.q * per_q;
    tp.b = rest / g.ncb;
    const int64_t cb = rest - tp.b * g.ncb;
    if (CHANNEL_LANES) {
        tp.j = cb * 64 + lane;
        tp.sub = w;
        tp.nsub = NW;
    } else {
        tp.j = cb;
        tp.sub = tid;
        tp.nsub = NT;
    }
    tp.ok = tp.j < g.H;
    tp.pos0 = tp.q * T + (int64_t)tp.sub * C;

    typename Op::Elem e[C];
    const Map m = op.template phase1<C>(tp, e);

    // exclusive prefix of this sub-chunk inside the chunk, and chunk aggregate
    Map ex, tot;
    if (CHANNEL_LANES) {
        s_part[w * 64 + lane] = m;
        __syncthreads();
        ex = M::id();
        for (int k = 0; k < w; ++k) ex = M::then(ex, s_part[k * 64 + lane]);
        tot = M::then(ex, m);
    } else {
        Map incl = m;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const Map o = M::shfl_up(incl, d);
            if (lane >= d) incl = M::then(o, incl);
        }
        Map exw = M::shfl_up(incl, 1);
        if (lane == 0) exw = M::id();
        if (lane == 63) s_part[w] = incl;
        __syncthreads();
        Map pre = M::id();
        for (int k = 0; k < w; ++k) pre = M::then(pre, s_part[k]);
        ex = M::then(pre, exw);
        tot = M::then(pre, incl);
    }

    // the holder of the chunk aggregate publishes it, looks back, and
    // publishes the state leaving the chunk
    const bool holder = CHANNEL_LANES ? (w == NW - 1) : (tid == NT - 1);
    if (holder) {
        State xin = op.init_state(tp);
        if (tp.ok) {
            const int64_t stride = g.B * g.H;
            const int64_t slot = tp.b * g.H + tp.j;
            const int64_t dsc = tp.q * stride + slot;
            if (tp.q > 0) {
                D::put_agg(g.agg + dsc * D::kAggWords, tot);
                xin = lookback<S>(g.agg, g.inc, tp.q, stride, slot, g.err);
            }
            D::put_inc(g.inc + dsc * D::kIncWords, M::apply(tot, xin));
            if (g.agg_next) {
                for (int k = 0; k < D::kAggWords; ++k) g.agg_next[dsc * D::kAggWords + k] = kSentinel64;
                for (int k = 0; k < D::kIncWords; ++k) g.inc_next[dsc * D::kIncWords + k] = kSentinel64;
            }
        }
        s_carry[CHANNEL_LANES ? lane : 0] = xin;
    }
    __syncthreads();
    const State x = M::apply(ex, s_carry[CHANNEL_LANES ? lane : 0]);
    op.template phase2<C, NW, CHANNEL_LANES>(tp, e, x);
}

// Reduce a per-thread value over the workgroup into one value per channel
// lane (channel lanes: sum over the waves of each lane; time lanes: sum over
// every thread).  Returns the total in wave 0 (lane = channel, or lane 0).
template <int NW, bool CHANNEL_LANES>
__device__ __forceinline__ float wg_channel_sum(float v, float *red /* shared, NW*64 */) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (!CHANNEL_LANES) v = wave_sum(v);
    red[w * 64 + lane] = v;
    __syncthreads();
    float s = 0.0f;
    if (w == 0) {
        if (CHANNEL_LANES) {
            for (int k = 0; k < NW; ++k) s += red[k * 64 + lane];
        } else {
            for (int k = 0; k < NW; ++k) s += red[k * 64];
        }
    }
    __syncthreads();
    return s;
}

}  // namespace prn
