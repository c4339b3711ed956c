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
#include "launch.hpp"

namespace prn {

struct ScanGeo {
    int64_t B, L, H;
    int64_t ncb;            // channel blocks per batch row (channel lanes: ceil(H/64); time lanes: H)
    int64_t nq;             // chunks along the sequence
    int64_t ntiles;         // workgroups of the launch (= tickets drawn)
    WsSpan ws;              // the caller's workspace: ticket header, size, what a wrap clear keeps
    uint64_t *agg, *inc;    // look-back descriptors [nq][B][H] (words per descriptor: Desc<S>)
};

// The span of a caller's workspace, keeping bytes [keep_lo, keep_hi) at the
// clear that ends a tag period (common.hpp, finish_launch).
inline WsSpan ws_span(const Ws &w, size_t keep_lo = 0, size_t keep_hi = 0) {
    return {reinterpret_cast<uint64_t *>(w.p), (uint64_t)(w.bytes / 8), (uint64_t)(keep_lo / 8),
            (uint64_t)(keep_hi / 8)};
}

struct TilePos {
    int64_t tile;           // workgroup ticket: (q * B + b) * ncb + channel block
    int64_t b, j, q, pos0;  // batch row, channel, chunk index, first position of this thread
    int sub, nsub;          // sub-chunk index of this thread within the chunk, and count
    bool ok;                // channel exists (j < H)
};

// ---------------------------------------------------------------- look-back
// Partial result of looking back over a run of consecutive predecessors,
// ordered nearest first: either the state entering the run's nearest end is
// known (found: x), or only the composite map of the whole run is (acc maps
// the state entering the run's farthest chunk to the state leaving its
// nearest one).  combine(near, far) is associative, so partials can be
// folded in any grouping as long as near stays before far.
template <int S> struct LbPart {
    typename MonoidT<S>::Map acc;
    typename MonoidT<S>::State x;
    int found;
};

template <int S>
__device__ __forceinline__ LbPart<S> lb_identity() {
    return {MonoidT<S>::id(), MonoidT<S>::zero(), 0};
}

template <int S>
__device__ __forceinline__ LbPart<S> lb_combine(const LbPart<S> &near, const LbPart<S> &far) {
    using M = MonoidT<S>;
    if (near.found) return near;
    LbPart<S> r;
    if (far.found) {
        r.found = 1;
        r.x = M::apply(near.acc, far.x);
        r.acc = near.acc;
    } else {
        r.found = 0;
        r.acc = M::then(far.acc, near.acc);
        r.x = far.x;
    }
    return r;
}

__device__ __forceinline__ float shfl_down_f(float v, int d) { return __shfl_down(v, d, 64); }
__device__ __forceinline__ Aff1 shfl_down_m(Aff1 m, int d) { return {shfl_down_f(m.a, d), shfl_down_f(m.b, d)}; }
__device__ __forceinline__ Aff2 shfl_down_m(Aff2 m, int d) {
    return {shfl_down_f(m.a00, d), shfl_down_f(m.a01, d), shfl_down_f(m.a10, d),
            shfl_down_f(m.a11, d), shfl_down_f(m.b0, d),  shfl_down_f(m.b1, d)};
}
__device__ __forceinline__ float shfl_down_s(float x, int d) { return shfl_down_f(x, d); }
__device__ __forceinline__ float2s shfl_down_s(float2s x, int d) {
    return {shfl_down_f(x.x, d), shfl_down_f(x.y, d)};
}

template <int K>
__device__ __forceinline__ AffK<K> shfl_down_m(const AffK<K> &m, int d) {
    AffK<K> r;
#pragma unroll
    for (int i = 0; i < K * K; ++i) r.a[i] = shfl_down_f(m.a[i], d);
#pragma unroll
    for (int i = 0; i < K; ++i) r.b[i] = shfl_down_f(m.b[i], d);
    return r;
}
template <int K>
__device__ __forceinline__ VecK<K> shfl_down_s(const VecK<K> &x, int d) {
    VecK<K> r;
#pragma unroll
    for (int i = 0; i < K; ++i) r.v[i] = shfl_down_f(x.v[i], d);
    return r;
}

__device__ __forceinline__ float bcast0_f(float v) { return __shfl(v, 0, 64); }
__device__ __forceinline__ Aff1 bcast0_m(Aff1 m) { return {bcast0_f(m.a), bcast0_f(m.b)}; }
__device__ __forceinline__ Aff2 bcast0_m(Aff2 m) {
    return {bcast0_f(m.a00), bcast0_f(m.a01), bcast0_f(m.a10), bcast0_f(m.a11), bcast0_f(m.b0), bcast0_f(m.b1)};
}
template <int K>
__device__ __forceinline__ AffK<K> bcast0_m(const AffK<K> &m) {
    AffK<K> r;
#pragma unroll
    for (int i = 0; i < K * K; ++i) r.a[i] = bcast0_f(m.a[i]);
#pragma unroll
    for (int i = 0; i < K; ++i) r.b[i] = bcast0_f(m.b[i]);
    return r;
}
template <int K>
__device__ __forceinline__ VecK<K> bcast0_s(const VecK<K> &x) {
    VecK<K> r;
#pragma unroll
    for (int i = 0; i < K; ++i) r.v[i] = bcast0_f(x.v[i]);
    return r;
}
__device__ __forceinline__ float bcast0_s(float x) { return bcast0_f(x); }
__device__ __forceinline__ float2s bcast0_s(float2s x) { return {bcast0_f(x.x), bcast0_f(x.y)}; }

// Descriptors polled per batch by one channel lane (channel lanes; fewer for
// the 2x2 blocks, whose descriptors are four times larger, to bound the
// registers held across the wait), and the window of the holder wave (time
// lanes: lane i polls predecessor i).
template <int S> constexpr int kLbBatch = S == 1 ? kLbBatchDiag : kLbBatchBlk2;

// Poll up to R consecutive predecessors p0, p0-1, ... (those >= 0) of one
// channel, issuing all loads before looking at any, and fold them nearest
// first until an inclusive state is met.  *next receives the first
// predecessor not folded (-1 once an inclusive state was found); a
// predecessor that has published nothing yet stops the fold there, to be
// polled again by the caller.
template <int S, int R>
__device__ __forceinline__ LbPart<S> lb_poll_batch(const ScanGeo &g, uint32_t tag, int64_t p0,
                                                   int64_t stride, int64_t slot, int64_t *next) {
    using M = MonoidT<S>;
    using D = Desc<S>;
    typename M::State xs[R];
    typename M::Map ms[R];
    int st[R];  // 0 nothing published, 1 aggregate, 2 inclusive, 3 before chunk 0
#pragma unroll
    for (int k = 0; k < R; ++k) {
        st[k] = 3;
        const int64_t p = p0 - k;
        if (p >= 0) {
            const int64_t d = p * stride + slot;
            const bool hi = D::get_inc(g.inc + d * D::kIncWords, xs[k], tag);
            const bool ha = D::get_agg(g.agg + d * D::kAggWords, ms[k], tag);
            st[k] = hi ? 2 : (ha ? 1 : 0);
        }
    }
    LbPart<S> part = lb_identity<S>();
    *next = p0 - R;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        if (part.found || *next != p0 - R) continue;
        if (st[k] == 2) {
            part = lb_combine<S>(part, LbPart<S>{M::id(), xs[k], 1});
            *next = -1;
        } else if (st[k] == 1) {
            part = lb_combine<S>(part, LbPart<S>{ms[k], M::zero(), 0});
        } else if (st[k] == 0) {
            *next = p0 - k;  // not published yet: resume here
        }
    }
    return part;
}

// State entering chunk q > 0 of one channel: batched, decoupled look-back by
// one lane.  Every predecessor holds a smaller ticket, so it is resident and
// publishes; the wait is still bounded (kMaxPolls rounds without progress
// give NaN).
template <int S>
__device__ typename MonoidT<S>::State lane_lookback(const ScanGeo &g, uint32_t tag, int64_t q,
                                                    int64_t stride, int64_t slot) {
    using M = MonoidT<S>;
    typename M::Map acc = M::id();  // state entering the farthest folded chunk -> entering q
    int64_t p = q - 1;
    uint32_t idle = 0;
    for (;;) {
        int64_t next;
        const LbPart<S> part = lb_poll_batch<S, kLbBatch<S>>(g, tag, p, stride, slot, &next);
        if (part.found) return M::apply(acc, part.x);
        acc = M::then(part.acc, acc);
        if (next == p) {
            if (++idle >= kMaxPolls) return nan_state<S>();
            __builtin_amdgcn_s_sleep(1);
        } else {
            idle = 0;
        }
        p = next;
    }
}

// State entering chunk q > 0 for a time-lane workgroup (one channel): the
// holder wave polls a window of 64 predecessors at once (lane i polls
// q-1-i), folds it with shuffles, and repeats with the next window until an
// inclusive state is met.  Called by every lane of one wave.
template <int S>
__device__ typename MonoidT<S>::State wave_lookback(const ScanGeo &g, uint32_t tag, int64_t q,
                                                    int64_t stride, int64_t slot) {
    using M = MonoidT<S>;
    using D = Desc<S>;
    const int lane = threadIdx.x & 63;
    typename M::Map acc_total = M::id();
    for (int64_t pbase = q - 1;; pbase -= 64) {
        const int64_t p = pbase - lane;
        LbPart<S> part = lb_identity<S>();
        if (p >= 0) {
            const int64_t d = p * stride + slot;
            for (uint32_t polls = 0;; ++polls) {
                typename M::State x;
                typename M::Map m;
                if (D::get_inc(g.inc + d * D::kIncWords, x, tag)) { part = {M::id(), x, 1}; break; }
                if (D::get_agg(g.agg + d * D::kAggWords, m, tag)) { part = {m, M::zero(), 0}; break; }
                if (polls >= kMaxPolls) {
                    part = {M::id(), nan_state<S>(), 1};
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            LbPart<S> far;
            far.acc = shfl_down_m(part.acc, d);
            far.x = shfl_down_s(part.x, d);
            far.found = __shfl_down(part.found, d, 64);
            if (lane + d < 64) part = lb_combine<S>(part, far);
        }
        // lane 0 holds the fold of the whole window; broadcast it
        if (__shfl(part.found, 0, 64)) return M::apply(acc_total, bcast0_s(part.x));
        acc_total = M::then(bcast0_m(part.acc), acc_total);
    }
}

// One tile (chunk q of a batch row and channel block, identified by its
// ticket) of a scan.  Every thread of the workgroup calls this.  With
// channel lanes the NW waves form NWC channel groups of 64 channels times
// NW/NWC sub-chunks, so a tile is 64*NWC channels wide (wider row segments
// per position) and (NW/NWC)*C positions long.
template <class Op, int NW, int C, bool CHANNEL_LANES, int NWC = 1>
__device__ __forceinline__ void scan_tile(const Op &op, const ScanGeo &g, int64_t ticket,
                                          uint32_t tag) {
    constexpr int S = Op::S;
    using M = MonoidT<S>;
    using D = Desc<S>;
    using Map = typename M::Map;
    using State = typename M::State;
    constexpr int NT = NW * 64;
    static_assert(NW % NWC == 0 && (CHANNEL_LANES || NWC == 1), "channel groups tile the waves");
    constexpr int NWT = NW / NWC;  // sub-chunks per chunk (channel lanes)
    constexpr int64_t T = CHANNEL_LANES ? (int64_t)NWT * C : (int64_t)NT * C;

    __shared__ Map s_part[CHANNEL_LANES ? NT : NW];
    __shared__ State s_carry[CHANNEL_LANES ? 64 * NWC : 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cw = w % NWC, tw = w / NWC;  // channel group, sub-chunk (channel lanes)
    const int64_t per_q = g.B * g.ncb;

    TilePos tp;
    tp.tile = ticket;
    tp.q = ticket / per_q;
    const int64_t rest = ticket - tp.q * per_q;
    tp.b = rest / g.ncb;
    const int64_t cb = rest - tp.b * g.ncb;
    if (CHANNEL_LANES) {
        tp.j = (cb * NWC + cw) * 64 + lane;
        tp.sub = tw;
        tp.nsub = NWT;
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
        for (int k = 0; k < tw; ++k) ex = M::then(ex, s_part[(k * NWC + cw) * 64 + lane]);
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

    // The holder of the chunk aggregate publishes it, finds the state
    // entering the chunk by look-back (per channel lane, or by the holder's
    // whole wave for time lanes) and publishes the state leaving the chunk.
    const bool holder = CHANNEL_LANES ? (tw == NWT - 1) : (tid == NT - 1);
    const int cslot = CHANNEL_LANES ? cw * 64 + lane : 0;
    const int64_t stride = g.B * g.H, slot = tp.b * g.H + tp.j;
    const int64_t dsc = tp.q * stride + slot;
    if (tp.q == 0) {
        if (holder) {
            const State xin = op.init_state(tp);
            if (tp.ok) D::put_inc(g.inc + dsc * D::kIncWords, M::apply(tot, xin), tag);
            s_carry[cslot] = xin;
        }
    } else if (CHANNEL_LANES) {
        if (holder) {
            State xin = M::zero();
            if (tp.ok) {
                D::put_agg(g.agg + dsc * D::kAggWords, tot, tag);
                xin = lane_lookback<S>(g, tag, tp.q, stride, slot);
                D::put_inc(g.inc + dsc * D::kIncWords, M::apply(tot, xin), tag);
            }
            s_carry[cslot] = xin;
        }
    } else if (w == NW - 1) {
        if (holder) D::put_agg(g.agg + dsc * D::kAggWords, tot, tag);
        const State xin = wave_lookback<S>(g, tag, tp.q, stride, slot);
        if (holder) {
            D::put_inc(g.inc + dsc * D::kIncWords, M::apply(tot, xin), tag);
            s_carry[0] = xin;
        }
    }
    __syncthreads();
    const State x = M::apply(ex, s_carry[cslot]);
    op.template phase2<C, NW, CHANNEL_LANES>(tp, e, x);
}

// One launch of a scan.  Tiles are handed out in the order of dynamically
// drawn tickets, which is what makes the look-back wait finite: a tile only
// waits for tiles with smaller tickets, whose workgroups are already running.
// With a grid of one workgroup per tile each workgroup draws one ticket.
// With a smaller (persistent) grid each workgroup keeps drawing until it
// draws past the last tile, so a launch draws ntiles + gridDim.x tickets and
// the last of them resets the header.  A tile ticket beyond the grid can only
// come from a workspace that was not zero-filled before its first use; such a
// workgroup does nothing.
template <class Op, int NW, int C, bool CHANNEL_LANES, int NWC = 1>
__global__ __launch_bounds__(NW * 64) void chunk_scan_kernel(Op op, ScanGeo g) {
    __shared__ Ticket s_ticket;
    if (!op.active()) return;  // uniform over the grid (e.g. Newton already converged)
    const bool persistent = (int64_t)gridDim.x < g.ntiles;
    const uint32_t draws = (uint32_t)(persistent ? g.ntiles + gridDim.x : g.ntiles);
    for (;;) {
        if (threadIdx.x == 0) s_ticket = draw_ticket(g.ws.hdr, draws);
        __syncthreads();  // scan_tile's own barriers keep the next write after every read
        const Ticket t = s_ticket;
        if (t.index >= g.ntiles) {
            finish_launch(t, g.ws);
            return;
        }
        scan_tile<Op, NW, C, CHANNEL_LANES, NWC>(op, g, t.index, t.tag);
        if (!persistent) {
            finish_launch(t, g.ws);
            return;
        }
    }
}

// Workgroups of a scan launch: one per tile, or with kScanPersistent as many
// as fit on the device at once (fewer workgroups to dispatch, which matters
// most for the Newton launches that find the iteration already converged
// and exit at once).
template <class Op, int NW, int C, bool CL, int NWC>
static int64_t scan_grid(int64_t ntiles) {
    if (!kScanPersistent) return ntiles;
    static const int per_cu =
        blocks_per_cu(reinterpret_cast<const void *>(chunk_scan_kernel<Op, NW, C, CL, NWC>), NW * 64);
    const int64_t slots = (int64_t)per_cu * device_cu_count();
    return ntiles < slots ? ntiles : slots;
}

template <class Op, int NW, int C, bool CL, int NWC = 1>
static hipError_t launch_chunk_scan(const Op &op, const ScanGeo &g, hipStream_t s) {
    const int64_t grid = scan_grid<Op, NW, C, CL, NWC>(g.ntiles);
    hipLaunchKernelGGL((chunk_scan_kernel<Op, NW, C, CL, NWC>), dim3((unsigned)grid), dim3(NW * 64), 0, s, op, g);
    return hipGetLastError();
}

}  // namespace prn
