// newton_chain.hip -- Newton's method for sequences longer than one workgroup
// holds, with every chunk kept on chip for all of its iterations (ParaRNN
// page, Fig. 5: the fully fused modality, extended here past one
// workgroup's reach).
//
// A tile is one chunk of T positions (of 64 channels, or of one channel for
// small H).  Its workgroup loads the gate inputs once and then runs Newton
// iterations k = 1, 2, ... on registers:
//   - the state before the chunk at iterate k-1 (h0 for the first chunk)
//     is kept on chip: zero at iterate 0, then advanced at every iteration
//     by the delta that enters the chunk, which is the previous chunk's
//     inclusive delta and so its last position's update;
//   - the cells give J_t and beta_t = F_t - s_t, composed per sub-chunk and
//     scanned inside the workgroup;
//   - the delta entering the chunk at iteration k comes from a decoupled
//     look-back over the previous chunks' iteration-k records;
//   - s += delta, and the chunk publishes its iteration-k records (aggregate
//     and inclusive delta).
// A chunk stops after iteration k once max|delta| <= tol over it and every
// chunk before it (a prefix AND of per-chunk flags, found by a second
// look-back), so the last chunk stops exactly when global Newton over the
// sequence would.  A stopped chunk's states are frozen: later iterations of
// its successors take a zero delta from it, so their copy of its last state
// stays put.  With tol = 0 no chunk stops before the cap and every iterate
// equals global Newton's (up to rounding: the state before a chunk is the sum
// of the deltas that entered it, which equals the previous chunk's stored
// last state in exact arithmetic).
//
// Every wait is on a chunk with a smaller ticket, whose workgroup is already
// running (tickets are drawn by running workgroups, in sequence order), so
// the waits end; they are bounded anyway (kMaxPolls, then NaN).
// The records of each iteration live in their own slice of the workspace,
// written once per launch with launch tags (common.hpp); a chunk may run
// several iterations ahead of its successor.
#include "cells.hpp"
#include "launch.hpp"
#include "scan_core.hpp"

namespace prn {

struct ChainGeo {
    int64_t B, L, H, ncb, nq, ntiles, ndesc;
    int32_t cap;
    float tol;
    WsSpan ws;                  // the caller's workspace (ticket header first)
    uint64_t *agg, *inc;        // [cap][ndesc][words]: iteration k at slice k-1
    uint64_t *stop;             // [ntiles]: last iteration of the tile (tagged)
    uint64_t *fagg, *finc;      // [cap][ntiles]: converged flag of the tile, and of it and all before it
    int32_t *info;
    uint32_t *trace;
};

// ---------------------------------------------------------------- cells
namespace {
constexpr float kE1 = -kLog2e, kE2 = -2.0f * kLog2e;
}

// GRU-style cell on pre-scaled gate inputs (pz, pr by -log2 e, pc by
// -2 log2 e), the same arithmetic as the fused kernel.
struct GruChain {
    static constexpr int S = 1, NG = 3;
    static constexpr bool kZeroMapOutside = false;  // positions outside are masked
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0;
    const float *h_init;  // initial iterate [B, L, H], or null for zeros
    float *h;
    bool runs;  // H == 1 with 16-byte aligned rows: whole runs move as float4

    using W = GruScaledW;
    __device__ W weights(int64_t j, bool ok) const {
        return ok ? gru_scaled_weights(uz[j], ur[j], uc[j]) : gru_scaled_weights(0.0f, 0.0f, 0.0f);
    }
    __device__ float init(int64_t b, int64_t j, int64_t H) const {
        return h0 != nullptr ? h0[b * H + j] : 0.0f;
    }
    __device__ bool warm() const { return h_init != nullptr; }
    // element e of the initial iterate (warm starts only)
    __device__ float guess(int64_t e) const { return h_init[e]; }
    template <int C>
    __device__ void load(int64_t base, int64_t H, const bool (&val)[C], bool whole, float (&x)[NG][C]) const {
        if constexpr (C % 4 == 0) {
            if (runs && whole) {
                load_run<C>(pz + base, x[0]);  // ordinary loads: streamed 16-byte
                load_run<C>(pr + base, x[1]);  // pieces of half-lines measured slower
                load_run<C>(pc + base, x[2]);
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    x[0][i] *= kE1;
                    x[1][i] *= kE1;
                    x[2][i] *= kE2;
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            // every load issued, none behind a branch (a position outside
            // reads element 0), so they are all in flight together
            const int64_t e = val[i] ? base + i * H : 0;
            x[0][i] = ld_once(pz + e);
            x[1][i] = ld_once(pr + e);
            x[2][i] = ld_once(pc + e);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x[0][i] = val[i] ? kE1 * x[0][i] : 0.0f;
            x[1][i] = val[i] ? kE1 * x[1][i] : 0.0f;
            x[2][i] = val[i] ? kE2 * x[2][i] : 0.0f;
        }
    }
    // Newton map of one position: delta -> J delta + (F - s), F and J at hp.
    __device__ Aff1 step(const W &w, float hp, float xz, float xr, float xc, float s) const {
        Aff1 m;
        gru_map_scaled(w, hp, xz, xr, xc, s, m.a, m.b);
        return m;
    }
    // step at hp = 0 and s = 0 (the first iteration from the zero iterate)
    __device__ Aff1 step0(const W &w, float xz, float xr, float xc) const {
        Aff1 m;
        gru_map_scaled0(w, xz, xr, xc, m.a, m.b);
        return m;
    }
    template <int C>
    __device__ void store(int64_t base, int64_t H, const bool (&val)[C], bool whole, const float (&s)[C]) const {
        if constexpr (C % 4 == 0) {
            if (runs && whole) {
                store_run<C>(h + base, s);
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < C; ++i)
            if (val[i]) h[base + i * H] = s[i];
    }
};

// LSTM-style cell; state (c, h) as (x, y).
struct LstmChain {
    static constexpr int S = 2, NG = 4;
    static constexpr bool kZeroMapOutside = true;  // see load()
    const float *pi, *pf, *po, *pg, *ui, *uf, *uo, *ug, *h0, *c0;
    const float *h_init, *c_init;  // initial iterates [B, L, H]; a null one is zero
    float *h, *c;
    bool runs;  // unused: the LSTM moves scalars

    struct W {
        float ui, uf, uo, ug;      // as given (the Jacobian)
        float uis, ufs, uos, ugs;  // pre-scaled as the gate inputs (the gates)
    };
    __device__ W weights(int64_t j, bool ok) const {
        W w{0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (ok) {
            w.ui = ui[j];
            w.uf = uf[j];
            w.uo = uo[j];
            w.ug = ug[j];
            w.uis = kE1 * w.ui;
            w.ufs = kE1 * w.uf;
            w.uos = kE1 * w.uo;
            w.ugs = kE2 * w.ug;
        }
        return w;
    }
    __device__ float2s init(int64_t b, int64_t j, int64_t H) const {
        return {c0 != nullptr ? c0[b * H + j] : 0.0f, h0 != nullptr ? h0[b * H + j] : 0.0f};
    }
    __device__ bool warm() const { return h_init != nullptr || c_init != nullptr; }
    __device__ float2s guess(int64_t e) const {
        return {c_init != nullptr ? c_init[e] : 0.0f, h_init != nullptr ? h_init[e] : 0.0f};
    }
    template <int C>
    __device__ void load(int64_t base, int64_t H, const bool (&val)[C], bool, float (&x)[NG][C]) const {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            // every load issued, none behind a branch (a position outside
            // reads element 0), so they are all in flight together
            const int64_t e = val[i] ? base + i * H : 0;
            x[0][i] = ld_once(pi + e);
            x[1][i] = ld_once(pf + e);
            x[2][i] = ld_once(po + e);
            x[3][i] = ld_once(pg + e);
        }
        // A position outside takes i = f = o = 0 (pre-scaled input +inf:
        // exp2 gives +inf, the reciprocal 0), which makes its Newton map
        // exactly zero (J = 0, F - s = 0 - 0), so its delta is 0 and
        // max|delta| needs no mask (kZeroMapOutside).
        constexpr float kOff = __builtin_inff();
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x[0][i] = val[i] ? kE1 * x[0][i] : kOff;
            x[1][i] = val[i] ? kE1 * x[1][i] : kOff;
            x[2][i] = val[i] ? kE1 * x[2][i] : kOff;
            x[3][i] = val[i] ? kE2 * x[3][i] : 0.0f;
        }
    }
    // Newton map of one position on the pre-scaled gate inputs (pi, pf, po by
    // -log2 e, pg by -2 log2 e): the arithmetic of lstm_f_j in cells.hpp with
    // each gate's pre-activation one fma in the exp2 domain, and the
    // derivative terms rewritten on products the cell already forms
    // (ig = i g, otc = o tanh c), each one multiply-add:
    //   g i(1-i) = ig - ig i,  i(1-g^2) = i - ig g,
    //   o(1-tanh^2 c) = o - otc tanh c,  o(1-o) tanh c = otc - otc o.
    __device__ Aff2 step(const W &w, float2s hp, float xi, float xf, float xo, float xg, float2s s) const {
        const float h = hp.y, cp = hp.x;
        const float i = fast_rcp(1.0f + fast_exp2(fmaf(w.uis, h, xi)));
        const float f = fast_rcp(1.0f + fast_exp2(fmaf(w.ufs, h, xf)));
        const float o = fast_rcp(1.0f + fast_exp2(fmaf(w.uos, h, xo)));
        const float g = fmaf(2.0f, fast_rcp(1.0f + fast_exp2(fmaf(w.ugs, h, xg))), -1.0f);
        const float ig = i * g;
        const float c = fmaf(f, cp, ig);
        const float tc = fmaf(2.0f, fast_rcp(1.0f + fast_exp2(kE2 * c)), -1.0f);
        const float otc = o * tc;
        const float odtc = fmaf(-otc, tc, o);
        const float kappa = fmaf(cp * fmaf(-f, f, f), w.uf, fmaf(fmaf(-ig, i, ig), w.ui, fmaf(-ig, g, i) * w.ug));
        return {f, kappa, odtc * f, fmaf(fmaf(-otc, o, otc), w.uo, odtc * kappa), c - s.x, otc - s.y};
    }
    template <int C>
    __device__ void store(int64_t base, int64_t H, const bool (&val)[C], bool, const float2s (&s)[C]) const {
#pragma unroll
        for (int i = 0; i < C; ++i)
            if (val[i]) {
                c[base + i * H] = s[i].x;
                h[base + i * H] = s[i].y;
            }
    }
};

template <class Cell, int C>
__device__ __forceinline__ typename MonoidT<Cell::S>::Map
cell_step(const Cell &cell, const typename Cell::W &w, typename MonoidT<Cell::S>::State hp,
          const float (&x)[Cell::NG][C], int i, typename MonoidT<Cell::S>::State s) {
    if constexpr (Cell::NG == 3)
        return cell.step(w, hp, x[0][i], x[1][i], x[2][i], s);
    else
        return cell.step(w, hp, x[0][i], x[1][i], x[2][i], x[3][i], s);
}

// ---------------------------------------------------------------- records
// A state record read ahead of use: the loads are issued early (before the
// cells of an iteration) and only looked at when the value is needed, so
// their latency hides behind the arithmetic.  A record not yet published is
// then polled as usual.
template <int S>
struct Ahead {
    uint64_t w[S];
    __device__ void issue(const uint64_t *p) {
#pragma unroll
        for (int k = 0; k < S; ++k) w[k] = ld_coherent(p + k);
    }
    __device__ bool get(typename MonoidT<S>::State &x, uint32_t tag) const;
};
template <>
__device__ __forceinline__ bool Ahead<1>::get(float &x, uint32_t tag) const {
    if (!has_tag(w[0], tag)) return false;
    x = lo_f(w[0]);
    return true;
}
template <>
__device__ __forceinline__ bool Ahead<2>::get(float2s &x, uint32_t tag) const {
    if (!has_tag(w[0], tag) || !has_tag(w[1], tag)) return false;
    x = {lo_f(w[0]), lo_f(w[1])};
    return true;
}

__device__ __forceinline__ bool stopped_before(const ChainGeo &g, int64_t ptile, uint32_t tag, int k,
                                               int *at = nullptr) {
    const uint64_t w = ld_coherent(g.stop + ptile);
    if (!has_tag(w, tag)) return false;
    const int s = (int)lo_f(w);
    if (at != nullptr) *at = s;
    return s < k;
}

// Delta entering chunk q at iteration k for one channel lane.
template <int S>
__device__ typename MonoidT<S>::State chain_lane_lookback(const ChainGeo &g, uint32_t tag, int k,
                                                          int64_t q, int64_t b, int64_t cb,
                                                          int64_t slot, const Ahead<S> &ahead) {
    using M = MonoidT<S>;
    using D = Desc<S>;
    {
        typename M::State x;
        if (ahead.get(x, tag)) return x;  // the previous chunk's inclusive delta, read ahead
    }
    const size_t kofs = (size_t)(k - 1) * g.ndesc;
    const int64_t stride = g.B * g.H;
    typename M::Map acc = M::id();
    int64_t p = q - 1;
    uint32_t idle = 0;
    while (p >= 0) {
        const int64_t d = p * stride + slot;
        typename M::State x;
        typename M::Map m;
        if (D::get_inc(g.inc + (kofs + d) * D::kIncWords, x, tag)) return M::apply(acc, x);
        if (D::get_agg(g.agg + (kofs + d) * D::kAggWords, m, tag)) {
            acc = M::then(m, acc);
            --p;
            idle = 0;
            continue;
        }
        if (stopped_before(g, (p * g.B + b) * g.ncb + cb, tag, k)) break;  // frozen prefix: zero delta
        if (++idle >= kMaxPolls) return nan_state<S>();
        __builtin_amdgcn_s_sleep(1);
    }
    return M::apply(acc, M::zero());
}

// Time lanes: the holder wave polls 64 predecessors at once (lane i polls
// chunk q-1-i) and folds them with shuffles.  Called by every lane of one wave.
template <int S>
__device__ typename MonoidT<S>::State chain_wave_lookback(const ChainGeo &g, uint32_t tag, int k,
                                                          int64_t q, int64_t b, int64_t cb,
                                                          int64_t slot, const Ahead<S> &ahead) {
    using M = MonoidT<S>;
    using D = Desc<S>;
    const int lane = threadIdx.x & 63;
    const size_t kofs = (size_t)(k - 1) * g.ndesc;
    const int64_t stride = g.B * g.H;
    typename M::Map acc_total = M::id();
    for (int64_t pbase = q - 1;; pbase -= 64) {
        const int64_t p = pbase - lane;
        LbPart<S> part = {M::id(), M::zero(), 1};  // before chunk 0: zero delta
        typename M::State xa;
        if (p >= 0 && pbase == q - 1 && ahead.get(xa, tag)) {
            part = {M::id(), xa, 1};  // read ahead
        } else if (p >= 0) {
            const int64_t d = p * stride + slot;
            for (uint32_t polls = 0;; ++polls) {
                typename M::State x;
                typename M::Map m;
                if (D::get_inc(g.inc + (kofs + d) * D::kIncWords, x, tag)) { part = {M::id(), x, 1}; break; }
                if (D::get_agg(g.agg + (kofs + d) * D::kAggWords, m, tag)) { part = {m, M::zero(), 0}; break; }
                if (stopped_before(g, (p * g.B + b) * g.ncb + cb, tag, k)) { part = {M::id(), M::zero(), 1}; break; }
                if (polls >= kMaxPolls) {
                    part = {M::id(), nan_state<S>(), 1};
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
#pragma unroll
        for (int dd = 1; dd < 64; dd <<= 1) {
            LbPart<S> far;
            far.acc = shfl_down_m(part.acc, dd);
            far.x = shfl_down_s(part.x, dd);
            far.found = __shfl_down(part.found, dd, 64);
            if (lane + dd < 64) part = lb_combine<S>(part, far);
        }
        if (__shfl(part.found, 0, 64)) return M::apply(acc_total, bcast0_s(part.x));
        acc_total = M::then(bcast0_m(part.acc), acc_total);
    }
}

// Whether every chunk before q (same batch row and channel block) had
// max|delta| <= tol at iteration k.  Called by every lane of one wave: lane i
// polls chunk q-1-i for its prefix flag (inclusive), its own flag
// (aggregate) or a stop before k (frozen, so converged); the nearest
// inclusive answer and every own flag nearer than it decide, and a false
// own flag decides at once.
__device__ bool chain_flag_lookback(const ChainGeo &g, uint32_t tag, int k, int64_t q, int64_t b, int64_t cb,
                                    uint64_t ahead) {
    const int lane = threadIdx.x & 63;
    const size_t kofs = (size_t)(k - 1) * g.ntiles;
    for (int64_t pbase = q - 1;; pbase -= 64) {
        const int64_t p = pbase - lane;
        int st = 3;  // 0 own false, 1 own true, 2 prefix false, 3 prefix true (or before chunk 0)
        if (p >= 0 && pbase == q - 1 && has_tag(ahead, tag)) {
            st = lo_f(ahead) != 0.0f ? 3 : 2;  // read ahead
        } else if (p >= 0) {
            const int64_t pt = (p * g.B + b) * g.ncb + cb;
            for (uint32_t polls = 0;; ++polls) {
                const uint64_t wi = ld_coherent(g.finc + kofs + pt);
                if (has_tag(wi, tag)) {
                    st = lo_f(wi) != 0.0f ? 3 : 2;
                    break;
                }
                const uint64_t wa = ld_coherent(g.fagg + kofs + pt);
                if (has_tag(wa, tag)) {
                    st = lo_f(wa) != 0.0f ? 1 : 0;
                    break;
                }
                if (stopped_before(g, pt, tag, k)) {
                    st = 3;
                    break;
                }
                if (polls >= kMaxPolls) {
                    st = 2;  // gave up: report not converged
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        const uint64_t incl = __ballot(st >= 2);
        const uint64_t bad = __ballot(st == 0 || st == 2);
        if (incl != 0) {
            const int first = __ffsll((unsigned long long)incl) - 1;
            const uint64_t upto = first == 63 ? ~0ull : ((1ull << (first + 1)) - 1);
            return (bad & upto) == 0;
        }
        if (bad != 0) return false;
    }
}

__device__ __forceinline__ float2s shfl_up_s(float2s x, int d) {
    return {__shfl_up(x.x, d, 64), __shfl_up(x.y, d, 64)};
}
__device__ __forceinline__ float shfl_up_s(float x, int d) { return __shfl_up(x, d, 64); }

__device__ __forceinline__ uint32_t state_abs_max(float d) { return abs_bits(d); }
__device__ __forceinline__ uint32_t state_abs_max(float2s d) {
    const uint32_t a = abs_bits(d.x), b = abs_bits(d.y);
    return a > b ? a : b;
}
__device__ __forceinline__ float state_add(float a, float b) { return a + b; }
__device__ __forceinline__ float2s state_add(float2s a, float2s b) { return {a.x + b.x, a.y + b.y}; }

// ---------------------------------------------------------------- tile
// LOCAL: the workgroup also ran the previous chunk of this chain (see
// newton_local_kernel), so the previous chunk's inclusive deltas are in LDS
// (s_rec, two halves used by alternate chunks, iteration k at row k-1), and
// kprev/cprev hold its last iteration and whether it stopped converged;
// nothing goes through global memory.  Every thread reads the delta entering
// the chunk from the previous chunk's half itself, while the holder writes
// this chunk's into the other half, so no barrier is needed between them.
// CW (channel lanes): channels per wave row.  With CW = 32 a wave holds two
// sub-chunks of 32 channels (lanes 0-31 and 32-63), so a chain is 32
// channels wide (128-byte rows) and a small workgroup still covers a
// useful chunk; only the whole-chain form takes it.
template <class Cell, int NW, int C, bool CL, bool LOCAL = false, int CW = 64>
__device__ __forceinline__ void chain_tile(const Cell &cell, const ChainGeo &g, int64_t ticket, uint32_t tag,
                                           int &kprev, bool &cprev) {
    static_assert(!LOCAL || CL, "workgroups own whole chains only with channel lanes");
    static_assert(CW == 64 || (CW == 32 && LOCAL), "half-wave channel rows only for the whole-chain form");
    constexpr int SPW = CL ? 64 / CW : 1;  // sub-chunks per wave (channel lanes)
    constexpr int NS = NW * SPW;           // sub-chunks per chunk (channel lanes)
    constexpr int S = Cell::S;
    using M = MonoidT<S>;
    using D = Desc<S>;
    using Map = typename M::Map;
    using State = typename M::State;
    constexpr int NT = NW * 64;
    constexpr int64_t T = CL ? (int64_t)NS * C : (int64_t)NT * C;

    __shared__ Map s_part[CL ? NT : NW];
    __shared__ State s_carry[CL ? 64 : 1];
    __shared__ State s_last[CL ? NT : NW];
    __shared__ uint32_t s_wmax[NW];
    __shared__ int s_stop;
    constexpr int kRecHalf = kChainMaxCap * CW;
    __shared__ State s_rec[LOCAL ? 2 * kRecHalf : 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t per_q = g.B * g.ncb;
    const int64_t q = ticket / per_q;
    const int64_t rest = ticket - q * per_q;
    const int64_t b = rest / g.ncb;
    const int64_t cb = rest - b * g.ncb;
    const int ch = lane % CW;  // channel within the chain's block (channel lanes)
    const int64_t j = CL ? cb * CW + ch : cb;
    const int sub = CL ? w * SPW + lane / CW : tid;
    const bool ok = j < g.H;
    const int64_t pos0 = q * T + (int64_t)sub * C;
    const int64_t base = idx3(b, pos0, ok ? j : 0, g.L, g.H);
    const int64_t stride = g.B * g.H, slot = b * g.H + j;
    const int64_t dsc = q * stride + slot;
    const bool holder = CL ? (sub == NS - 1) : (tid == NT - 1);

    bool val[C];
#pragma unroll
    for (int i = 0; i < C; ++i) val[i] = ok && pos0 + i < g.L;
    const bool whole = ok && pos0 + C <= g.L;
    // time lanes: positions of this thread inside the sequence, the first nv
    int nv = ok ? (int)(g.L - pos0 < 0 ? 0 : g.L - pos0 < C ? g.L - pos0 : C) : 0;
    float x[Cell::NG][C];
    cell.template load<C>(base, g.H, val, whole, x);
    const typename Cell::W wts = cell.weights(j, ok);
    // iterate 0: zero, or the caller's initial iterate (a warm start)
    const bool warm = cell.warm();
    State s[C];
#pragma unroll
    for (int i = 0; i < C; ++i) s[i] = (warm && val[i]) ? cell.guess(base + i * g.H) : M::zero();
    const State init = (ok && q == 0 && sub == 0) ? cell.init(b, j, g.H) : M::zero();
    // The state before this chunk (the previous chunk's last state) at the
    // current iterate, kept by the sub-chunk-0 threads: its value at iterate
    // 0 (zero, or the initial iterate's), then advanced by the delta entering
    // the chunk at each iteration, which is the previous chunk's inclusive
    // delta (zero once that chunk has stopped).
    State hb = (warm && ok && q > 0 && sub == 0) ? cell.guess(base - g.H) : M::zero();

    int k = 1;
    bool conv = false;
    for (;; ++k) {
        const size_t kofs = (size_t)(k - 1) * g.ndesc;
        // Records of the previous chunk read ahead of the cells: its
        // inclusive delta and converged flag at k.
        Ahead<S> a_inc{};  // zero words never carry a launch tag
        uint64_t a_flag = 0;
        if (!LOCAL && q > 0) {
            if (CL ? (holder && ok) : (w == NW - 1 && q - 1 - lane >= 0))
                a_inc.issue(g.inc + (kofs + (CL ? dsc - stride : (q - 1 - lane) * stride + slot)) * D::kIncWords);
            if (w == 0 && q - 1 - lane >= 0)
                a_flag = ld_coherent(g.finc + (size_t)(k - 1) * g.ntiles + ((q - 1 - lane) * g.B + b) * g.ncb + cb);
        }

        // cells at iterate k-1: positions 1..C-1 first (their previous state
        // is this thread's own), then position 0, whose previous state may
        // come from the previous chunk
        // Every position is evaluated, with no branch per position, so the
        // compiler can interleave the independent cells.  A position past the
        // end of the sequence or a channel past H runs on inputs the cell
        // chooses (zero for the GRU; for the LSTM ones that make its map zero);
        // its map reaches only later positions of the same chunk (also past
        // the end), the records of the last chunk (which no chunk reads) and
        // states that are never stored (nor, for the GRU, counted in
        // max|delta|; the LSTM's are zero).
        Map e[C];
        const auto cells = [&]() {
#pragma unroll
            for (int i = 1; i < C; ++i) e[i] = cell_step<Cell, C>(cell, wts, s[i - 1], x, i, s[i]);
        };
        if constexpr (LOCAL && S == 1) {
            // From the zero iterate, positions 1.. see a zero previous state.
            // Only the GRU's whole-chain form takes this: in the other forms
            // the second copy of the cell loop costs registers, spills or
            // occupancy.
            if (k == 1 && !warm) {
#pragma unroll
                for (int i = 1; i < C; ++i) e[i] = cell.step0(wts, x[0][i], x[1][i], x[2][i]);
            } else {
                cells();
            }
        } else {
            cells();
        }
        State hp = M::zero();
        State nb = M::zero();
        if (!CL) nb = shfl_up_s(s[C - 1], 1);  // every lane active for the shuffle
        if (sub == 0) {
            hp = q == 0 ? init : hb;
        } else if (k > 1) {
            if (CL)
                hp = s_last[(sub - 1) * CW + ch];
            else
                hp = lane == 0 ? s_last[w - 1] : nb;
        } else if (warm && ok && pos0 <= g.L) {
            hp = cell.guess(base - g.H);  // iterate 0 before this sub-chunk
        }
        e[0] = cell_step<Cell, C>(cell, wts, hp, x, 0, s[0]);
        Map acc = e[0];
#pragma unroll
        for (int i = 1; i < C; ++i) acc = M::then(acc, e[i]);

        // exclusive prefix of this sub-chunk inside the chunk, and the chunk
        // aggregate; in the whole-chain form the delta entering the chunk is
        // already known, so each thread instead carries that delta through
        // the earlier sub-chunks' maps (a map applied to a state costs a third
        // of a map composed with a map, for 2x2 blocks) and nothing is composed
        Map ex, tot;
        State din_sub;  // whole-chain form: the delta entering this sub-chunk
        if (LOCAL) {
            s_part[sub * CW + ch] = acc;
            lds_barrier();
            Map pv[NS - 1];
#pragma unroll
            for (int kk = 0; kk < NS - 1; ++kk)
                if (kk < sub) pv[kk] = s_part[kk * CW + ch];
            // the previous chunk's inclusive delta at k (zero once it has
            // stopped)
            din_sub = (q > 0 && k <= kprev) ? s_rec[((q - 1) & 1) * kRecHalf + (k - 1) * CW + ch] : M::zero();
#pragma unroll
            for (int kk = 0; kk < NS - 1; ++kk)
                if (kk < sub) din_sub = M::apply(pv[kk], din_sub);
        } else if (CL) {
            s_part[sub * CW + ch] = acc;
            lds_barrier();
            // the earlier sub-chunks' maps are all read before any is
            // composed, so their LDS latencies overlap
            Map pv[NS - 1];
#pragma unroll
            for (int kk = 0; kk < NS - 1; ++kk)
                if (kk < sub) pv[kk] = s_part[kk * CW + ch];
            ex = sub > 0 ? pv[0] : M::id();
#pragma unroll
            for (int kk = 1; kk < NS - 1; ++kk)
                if (kk < sub) ex = M::then(ex, pv[kk]);
            tot = sub > 0 ? M::then(ex, acc) : acc;
        } else {
            Map incl = acc;
#pragma unroll
            for (int dd = 1; dd < 64; dd <<= 1) {
                const Map o = M::shfl_up(incl, dd);
                if (lane >= dd) incl = M::then(o, incl);
            }
            Map exw = M::shfl_up(incl, 1);
            if (lane == 0) exw = M::id();
            if (lane == 63) s_part[w] = incl;
            lds_barrier();
            Map pre = M::id();
            for (int kk = 0; kk < w; ++kk) pre = M::then(pre, s_part[kk]);
            ex = M::then(pre, exw);
            tot = M::then(pre, incl);
        }

        // delta entering the chunk at iteration k
        State cin;
        if (LOCAL) {
            // the holder records this chunk's inclusive delta for the next
            // chunk; only sub-chunk 0 needs the delta entering the chunk (hb)
            cin = din_sub;
            if (holder) s_rec[(q & 1) * kRecHalf + (k - 1) * CW + ch] = M::apply(acc, din_sub);
        } else if (CL) {
            if (holder) {
                State din = M::zero();
                if (ok) {
                    if (q > 0) {
                        D::put_agg(g.agg + (kofs + dsc) * D::kAggWords, tot, tag);
                        din = chain_lane_lookback<S>(g, tag, k, q, b, cb, slot, a_inc);
                    }
                    D::put_inc(g.inc + (kofs + dsc) * D::kIncWords, M::apply(tot, din), tag);
                }
                s_carry[lane] = din;
            }
        } else if (w == NW - 1) {
            State din = M::zero();
            if (q > 0) {
                if (holder) D::put_agg(g.agg + (kofs + dsc) * D::kAggWords, tot, tag);
                din = chain_wave_lookback<S>(g, tag, k, q, b, cb, slot, a_inc);
            }
            if (holder) {
                D::put_inc(g.inc + (kofs + dsc) * D::kIncWords, M::apply(tot, din), tag);
                s_carry[0] = din;
            }
        }
        if (!LOCAL) {
            lds_barrier();
            cin = s_carry[CL ? lane : 0];
        }

        // apply: delta through the sub-chunk, s += delta
        if (sub == 0) hb = state_add(hb, cin);  // the previous chunk's last state at iterate k
        State dlt = LOCAL ? din_sub : M::apply(ex, cin);
        uint32_t mx = 0;
        // max|delta| over the positions inside the sequence.  The LSTM needs
        // no mask (a position outside has a zero map, so a zero delta).  For
        // the GRU with time lanes, a thread whose positions all lie inside
        // (every thread but those of a chain's last chunk) takes no mask
        // either: the masks are lane masks in scalar registers, which that
        // kernel keeps spilled, so each masked position would cost two
        // reloads; the others test i < nv, which the empty asm makes opaque
        // so that the masks are not hoisted out of the loop and kept live
        // across it.  With channel lanes the split measured slower.
        if constexpr (!CL) asm volatile("" : "+v"(nv));
        const auto apply_all = [&](auto masked) {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                dlt = M::apply(e[i], dlt);
                s[i] = state_add(s[i], dlt);
                const bool in = CL ? val[i] : i < nv;
                const uint32_t a = (!decltype(masked)::value || in) ? state_abs_max(dlt) : 0u;
                mx = a > mx ? a : mx;
            }
        };
        if constexpr (Cell::kZeroMapOutside) {
            apply_all(std::false_type{});  // positions outside have delta 0
        } else {
            if (!CL && whole)
                apply_all(std::false_type{});
            else
                apply_all(std::true_type{});
        }
        mx = clamp_nan_to_inf(mx);
        if (CL)
            s_last[sub * CW + ch] = s[C - 1];
        else if (lane == 63)
            s_last[w] = s[C - 1];
        mx = wave_max_u32(mx);
        if (lane == 0) s_wmax[w] = mx;
        lds_barrier();
        uint32_t m = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) m = s_wmax[ww] > m ? s_wmax[ww] : m;
        // stop once this chunk and every chunk before it have converged
        if (LOCAL) {
            // every thread decides alike: the previous chunk counts as
            // converged from the iteration it stopped at, if it converged
            conv = __uint_as_float(m) <= g.tol && (q == 0 || (cprev && k >= kprev));
            if (tid == 0 && g.trace != nullptr) {
                const uint32_t cur = __hip_atomic_load(g.trace + (k - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (m > cur)
                    __hip_atomic_fetch_max(g.trace + (k - 1), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (conv || k >= g.cap) break;
            continue;
        }
        if (w == 0) {
            const bool own = __uint_as_float(m) <= g.tol;
            const size_t fofs = (size_t)(k - 1) * g.ntiles + ticket;
            if (lane == 0) {
                st_coherent(g.fagg + fofs, tagged(own ? 1.0f : 0.0f, tag));
                if (g.trace != nullptr) {
                    const uint32_t cur = __hip_atomic_load(g.trace + (k - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (m > cur)
                        __hip_atomic_fetch_max(g.trace + (k - 1), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            bool prefix = own;
            if (own && q > 0) prefix = chain_flag_lookback(g, tag, k, q, b, cb, a_flag);
            if (lane == 0) {
                if (own) st_coherent(g.finc + fofs, tagged(prefix ? 1.0f : 0.0f, tag));
                s_stop = prefix ? 1 : 0;
            }
        }
        if (__uint_as_float(m) > g.tol) {
            // every thread already knows this chunk has not converged: there
            // is no prefix decision to wait for (wave 0 published the flag)
            if (k >= g.cap) break;
            continue;
        }
        lds_barrier();
        conv = s_stop != 0;
        if (conv || k >= g.cap) break;
    }
    if (!LOCAL && tid == 0) st_coherent(g.stop + ticket, tagged((float)k, tag));
    kprev = k;
    cprev = conv;
    if constexpr (!CL) {
        asm volatile("" : "+v"(nv));
#pragma unroll
        for (int i = 0; i < C; ++i) val[i] = i < nv;
    }
    cell.template store<C>(base, g.H, val, whole, s);
    if (tid == 0 && g.info != nullptr) {
        if (k > __hip_atomic_load(g.info, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            __hip_atomic_fetch_max(g.info, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!conv && __hip_atomic_load(g.info + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
            __hip_atomic_store(g.info + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <class Cell, int NW, int C, bool CL>
__global__ __launch_bounds__(NW * 64, kChainMinWaves) void newton_chain_kernel(Cell cell, ChainGeo g) {
    __shared__ Ticket s_ticket;
    const bool persistent = (int64_t)gridDim.x < g.ntiles;
    const uint32_t draws = (uint32_t)(persistent ? g.ntiles + gridDim.x : g.ntiles);
    for (;;) {
        if (threadIdx.x == 0) s_ticket = draw_ticket(g.ws.hdr, draws);
        __syncthreads();
        const Ticket t = s_ticket;
        if (t.index >= g.ntiles) {
            finish_launch(t, g.ws);
            return;
        }
        int kprev = 0;
        bool cprev = false;
        chain_tile<Cell, NW, C, CL>(cell, g, t.index, t.tag, kprev, cprev);
        if (!persistent) {
            finish_launch(t, g.ws);
            return;
        }
        __syncthreads();  // the tile's last reads of shared memory before the next ticket
    }
}

// Workgroups that own whole chains (a chain: the chunks of one batch row and
// channel block): workgroup i runs chains i, i + grid, ... and each chain's
// chunks in order, so a chunk finds everything it needs from its predecessor
// in LDS and no workgroup waits on another.  The iterates equal those of the
// chained kernel above.  Worth it once there are at least as many chains as
// workgroup slots on the device.
template <class Cell, int NW, int C, int CW>
__global__ __launch_bounds__(NW * 64, kChainMinWaves) void newton_local_kernel(Cell cell, ChainGeo g) {
    const int64_t nchains = g.B * g.ncb;
    for (int64_t ch = blockIdx.x; ch < nchains; ch += gridDim.x) {
        int kprev = 0;
        bool cprev = false;
        for (int64_t q = 0; q < g.nq; ++q) {
            chain_tile<Cell, NW, C, true, true, CW>(cell, g, q * nchains + ch, 0u, kprev, cprev);
            __syncthreads();  // the chunk's last reads of shared memory before the next chunk
        }
    }
}

template <class Cell, int NW, int C, int CW>
static int64_t local_slots() {
    static const int per_cu =
        blocks_per_cu(reinterpret_cast<const void *>(newton_local_kernel<Cell, NW, C, CW>), NW * 64);
    return (int64_t)per_cu * device_cu_count();
}

template <class Cell, int NW, int C, int CW>
static hipError_t launch_local(const Cell &cell, const ChainGeo &g, hipStream_t s) {
    const int64_t slots = local_slots<Cell, NW, C, CW>(), nchains = g.B * g.ncb;
    const int64_t grid = nchains < slots ? nchains : slots;
    hipLaunchKernelGGL((newton_local_kernel<Cell, NW, C, CW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, cell, g);
    return hipGetLastError();
}

template <class Cell, int NW, int C, bool CL>
static hipError_t launch_chain(const Cell &cell, const ChainGeo &g, hipStream_t s) {
    static const int per_cu =
        blocks_per_cu(reinterpret_cast<const void *>(newton_chain_kernel<Cell, NW, C, CL>), NW * 64);
    const int64_t slots = (int64_t)per_cu * device_cu_count();
    const int64_t grid = g.ntiles < slots ? g.ntiles : slots;
    hipLaunchKernelGGL((newton_chain_kernel<Cell, NW, C, CL>), dim3((unsigned)grid), dim3(NW * 64), 0, s, cell, g);
    return hipGetLastError();
}

// Whether the chained forward lets workgroups own whole chains: always with
// local = 1 (and channel lanes), never with local = 0, and with local = -1
// when there are at least as many chains as workgroup slots for the kernel
// that owns them.  lcfg is the tile of that kernel (channel lanes).  The
// workspace query and the dispatch both decide with this function: the
// whole-chain form uses no workspace beyond the header.
template <class Cell, int NWL, int CLC, int CWL>
static bool owns_chains(const TileCfg &lcfg, int64_t B, int64_t L, int64_t H, int local) {
    if (H < kChannelLanesMinH || local == 0) return false;
    if (local > 0) return true;
    return B * scan_shape(lcfg, B, L, H).ncb >= local_slots<Cell, NWL, CLC, CWL>();
}

template <class Cell, int NWC, int CC, int NWT, int CT, int NWL, int CLC, int CWL>
static hipError_t chain_forward(const TileCfg &cfg, const TileCfg &lcfg, const Cell &cell, int64_t B, int64_t L,
                                int64_t H, int32_t cap, float tol, int32_t *info, float *trace, int local,
                                const Ws &ws, hipStream_t s) {
    FillRange fr[3] = {
        {info, info ? 1ull : 0ull, 0, 4},                         // iterations = 0
        {info ? info + 1 : nullptr, info ? 1ull : 0ull, 1, 4},    // converged = 1
        {trace, trace ? (uint64_t)cap : 0ull, 0, 4},
    };
    hipError_t e = fill(fr, 3, s);
    if (e != hipSuccess) return e;
    ChainGeo g;
    g.B = B;
    g.L = L;
    g.H = H;
    g.cap = cap;
    g.tol = tol;
    g.info = info;
    g.trace = reinterpret_cast<uint32_t *>(trace);
    g.ws = ws_span(ws);
    if (owns_chains<Cell, NWL, CLC, CWL>(lcfg, B, L, H, local)) {
        // no records, no tickets: the workspace is not touched
        const ScanShape ls = scan_shape(lcfg, B, L, H);
        g.ncb = ls.ncb;
        g.nq = ls.nq;
        g.ntiles = ls.ntiles;
        g.ndesc = ls.ndesc;
        g.agg = g.inc = g.stop = g.fagg = g.finc = nullptr;
        return launch_local<Cell, NWL, CLC, CWL>(cell, g, s);
    }
    const ChainWs w = chain_ws(cfg, Cell::S, B, L, H, cap);
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.ndesc = w.sh.ndesc;
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    g.stop = reinterpret_cast<uint64_t *>(ws.p + w.stop);
    g.fagg = reinterpret_cast<uint64_t *>(ws.p + w.fagg);
    g.finc = reinterpret_cast<uint64_t *>(ws.p + w.finc);
    if (!w.sh.channel_lanes) return launch_chain<Cell, NWT, CT, false>(cell, g, s);
    return launch_chain<Cell, NWC, CC, true>(cell, g, s);
}

bool gru_chain_owns_chains(int64_t B, int64_t L, int64_t H, int local) {
    constexpr TileCfg lc = kCfgGruLocal;
    return owns_chains<GruChain, lc.nw_cl, lc.c_cl, lc.cw_cl>(lc, B, L, H, local);
}

bool lstm_chain_owns_chains(int64_t B, int64_t L, int64_t H, int local) {
    constexpr TileCfg lc = kCfgLstmLocal;
    return owns_chains<LstmChain, lc.nw_cl, lc.c_cl, lc.cw_cl>(lc, B, L, H, local);
}

hipError_t gru_forward_chain(const GruFwdArgs &a, const Ws &ws, hipStream_t s) {
    GruChain cell;
    cell.pz = a.pz;
    cell.pr = a.pr;
    cell.pc = a.pc;
    cell.uz = a.uz;
    cell.ur = a.ur;
    cell.uc = a.uc;
    cell.h0 = a.h0;
    cell.h_init = a.h_init;
    cell.h = a.h;
    cell.runs = a.H == 1 && a.L % 4 == 0 && aligned16(a.pz) && aligned16(a.pr) && aligned16(a.pc) &&
                aligned16(a.h);
    constexpr TileCfg c = kCfgGruChain, lc = kCfgGruLocal;
    return chain_forward<GruChain, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, lc.nw_cl, lc.c_cl, lc.cw_cl>(
        c, lc, cell, a.B, a.L, a.H, a.cap, a.tol, a.info, a.trace, a.local, ws, s);
}

hipError_t lstm_forward_chain(const LstmFwdArgs &a, const Ws &ws, hipStream_t s) {
    LstmChain cell;
    cell.pi = a.pi;
    cell.pf = a.pf;
    cell.po = a.po;
    cell.pg = a.pg;
    cell.ui = a.ui;
    cell.uf = a.uf;
    cell.uo = a.uo;
    cell.ug = a.ug;
    cell.h0 = a.h0;
    cell.c0 = a.c0;
    cell.h_init = a.h_init;
    cell.c_init = a.c_init;
    cell.h = a.h;
    cell.c = a.c;
    cell.runs = false;
    constexpr TileCfg c = kCfgLstmChain, lc = kCfgLstmLocal;
    return chain_forward<LstmChain, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, lc.nw_cl, lc.c_cl, lc.cw_cl>(
        c, lc, cell, a.B, a.L, a.H, a.cap, a.tol, a.info, a.trace, a.local, ws, s);
}

}  // namespace prn
