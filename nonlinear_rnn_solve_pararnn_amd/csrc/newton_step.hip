// newton_step.hip -- Newton's method for the whole sequence with one launch
// per iteration (ParaRNN page, Fig. 5 caption: the modality that assembles
// the system and runs the parallel reduction as separate stages, here fused
// into one HBM pass).  The chained kernel (newton_chain.hip) is the default
// for long sequences; this path is selectable and takes caps above the
// chained kernel's limit.
//
// Iteration k (from s^0 = 0, or from the caller's initial iterate):
//   F_t = f(s^{k-1}_{t-1}), J_t = df/ds there, beta_t = F_t - s^{k-1}_t,
//   delta_t = J_t delta_{t-1} + beta_t (delta_{-1} = 0)  -- the bi-diagonal
//   solve, done by the chunked look-back scan,
//   s^k_t = s^{k-1}_t + delta_t,  e_k = max |delta| (NaN counts as +inf).
// One launch reads the gate inputs and s^{k-1} and writes s^k in place.  A
// chunk's first cell needs s^{k-1} at the end of the previous chunk, which
// that chunk's workgroup may already have overwritten in this launch, so the
// last state of every chunk is also kept in a small boundary array
// (alternating between two copies).  Every launch first reads e_{k-1}; once
// an iteration has met the tolerance every later launch exits at once, so
// the host can enqueue max_iter launches without waiting for the device.
// A warm start first copies the initial iterate into the outputs and its
// chunk-end states into the boundary array that iteration 1 reads; iteration
// 1 then runs as every later one.
#include <algorithm>

#include "cells.hpp"
#include "launch.hpp"
#include "newton_iter.hpp"
#include "scan_core.hpp"

namespace prn {

// ---------------------------------------------------------------- GRU
struct GruStepOp {
    static constexpr int S = 1;
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0;
    float *h;
    const float *bnd_prev;
    float *bnd_next;
    uint32_t *maxd;
    float tol;
    int k;
    bool cold1;  // iteration 1 from s^0 = 0 (no initial iterate)
    int64_t B, L, H;

    struct Elem {
        float J, beta, hc;
    };
    __device__ bool active() const { return newton_active(maxd, k, tol); }
    __device__ float init_state(const TilePos &) const { return 0.0f; }

    bool runs;  // H == 1 with 16-byte aligned rows: whole runs move as float4

    template <int C>
    __device__ Aff1 phase1(const TilePos &tp, Elem (&e)[C]) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        float hp = 0.0f;  // s^{k-1} at pos0 - 1
        float wz = 0.0f, wr = 0.0f, wc = 0.0f;
        if (tp.ok) {
            wz = uz[tp.j];
            wr = ur[tp.j];
            wc = uc[tp.j];
            if (tp.pos0 == 0)
                hp = h0 != nullptr ? h0[tp.b * H + tp.j] : 0.0f;
            else if (cold1)
                hp = 0.0f;
            else if (tp.sub == 0)
                hp = bnd_prev[(tp.q - 1) * B * H + tp.b * H + tp.j];
            else if (tp.pos0 <= L)  // a sub-chunk wholly past the end reads nothing
                hp = h[base - H];
        }
        Aff1 acc = {1.0f, 0.0f};
        if constexpr (C % 4 == 0) {
            if (runs && tp.ok && tp.pos0 + C <= L) {
                float vz[C], vr[C], vc[C], vh[C];
                load_run<C>(pz + base, vz);  // ordinary loads: streamed 16-byte
                load_run<C>(pr + base, vr);  // pieces of half-lines measured slower
                load_run<C>(pc + base, vc);
                if (cold1) {
#pragma unroll
                    for (int i = 0; i < C; ++i) vh[i] = 0.0f;
                } else {
                    load_run<C>(h + base, vh);
                }
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    float F, J;
                    gru_f_j(hp, vz[i], vr[i], vc[i], wz, wr, wc, F, J);
                    e[i] = {J, F - vh[i], vh[i]};
                    hp = vh[i];
                    acc = {acc.a * J, fmaf(J, acc.b, e[i].beta)};
                }
                return acc;
            }
        }
        const auto cell = [&](int i) {
            const int64_t kk = base + i * H;
            const float hc = cold1 ? 0.0f : h[kk];
            float F, J;
            gru_f_j(hp, ld_once(pz + kk), ld_once(pr + kk), ld_once(pc + kk), wz, wr, wc, F, J);
            e[i] = {J, F - hc, hc};
            hp = hc;
        };
        if (tp.ok && tp.pos0 + C <= L) {  // every position inside: no test per position
#pragma unroll
            for (int i = 0; i < C; ++i) {
                cell(i);
                acc = {acc.a * e[i].J, fmaf(e[i].J, acc.b, e[i].beta)};
            }
            return acc;
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if (tp.ok && tp.pos0 + i < L)
                cell(i);
            else
                e[i] = {1.0f, 0.0f, 0.0f};
            acc = {acc.a * e[i].J, fmaf(e[i].J, acc.b, e[i].beta)};
        }
        return acc;
    }

    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float d) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        uint32_t mx = 0;
        bool done = false;  // the workgroup reduction below must be reached by every thread
        if constexpr (C % 4 == 0) {
            if (runs && tp.ok && tp.pos0 + C <= L) {
                float hn[C];
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    d = fmaf(e[i].J, d, e[i].beta);
                    hn[i] = e[i].hc + d;
                    const uint32_t ad = abs_bits(d);
                    mx = ad > mx ? ad : mx;
                }
                store_run<C>(h + base, hn);
                if (tp.sub == tp.nsub - 1) bnd_next[tp.q * B * H + tp.b * H + tp.j] = hn[C - 1];
                done = true;
            }
        }
        const auto update = [&](int i) {
            d = fmaf(e[i].J, d, e[i].beta);
            const float hn = e[i].hc + d;
            h[base + i * H] = hn;
            const uint32_t ad = abs_bits(d);
            mx = ad > mx ? ad : mx;
            if (i == C - 1 && tp.sub == tp.nsub - 1) bnd_next[tp.q * B * H + tp.b * H + tp.j] = hn;
        };
        if (!done && tp.ok && tp.pos0 + C <= L) {
#pragma unroll
            for (int i = 0; i < C; ++i) update(i);
        } else if (!done) {
#pragma unroll
            for (int i = 0; i < C; ++i)
                if (tp.ok && tp.pos0 + i < L) update(i);
        }
        wg_max_to<NW>(mx, maxd + (k - 1));
    }
};

// ---------------------------------------------------------------- LSTM
// State (c, h); boundary arrays hold float2 (c, h).
struct LstmStepOp {
    static constexpr int S = 2;
    const float *pi, *pf, *po, *pg, *ui, *uf, *uo, *ug, *h0, *c0;
    float *h, *c;
    const float2 *bnd_prev;
    float2 *bnd_next;
    uint32_t *maxd;
    float tol;
    int k;
    bool cold1;  // iteration 1 from s^0 = 0 (no initial iterate)
    int64_t B, L, H;

    struct Elem {
        Aff2 m;       // J and beta
        float cc, hc; // s^{k-1}
    };
    __device__ bool active() const { return newton_active(maxd, k, tol); }
    __device__ float2s init_state(const TilePos &) const { return {0.0f, 0.0f}; }

    template <int C>
    __device__ Aff2 phase1(const TilePos &tp, Elem (&e)[C]) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        float cp = 0.0f, hp = 0.0f;
        float wi = 0.0f, wf = 0.0f, wo = 0.0f, wg = 0.0f;
        if (tp.ok) {
            wi = ui[tp.j];
            wf = uf[tp.j];
            wo = uo[tp.j];
            wg = ug[tp.j];
            if (tp.pos0 == 0) {
                hp = h0 != nullptr ? h0[tp.b * H + tp.j] : 0.0f;
                cp = c0 != nullptr ? c0[tp.b * H + tp.j] : 0.0f;
            } else if (cold1) {
            } else if (tp.sub == 0) {
                const float2 v = bnd_prev[(tp.q - 1) * B * H + tp.b * H + tp.j];
                cp = v.x;
                hp = v.y;
            } else if (tp.pos0 <= L) {  // a sub-chunk wholly past the end reads nothing
                cp = c[base - H];
                hp = h[base - H];
            }
        }
        Aff2 acc;
        const auto cell = [&](int i) {
            const int64_t kk = base + i * H;
            const float cc = cold1 ? 0.0f : c[kk];
            const float hc = cold1 ? 0.0f : h[kk];
            const Lstm2 r = lstm_f_j(cp, hp, ld_once(pi + kk), ld_once(pf + kk), ld_once(po + kk),
                                     ld_once(pg + kk), wi, wf, wo, wg);
            e[i].m = {r.j00, r.j01, r.j10, r.j11, r.Fc - cc, r.Fh - hc};
            e[i].cc = cc;
            e[i].hc = hc;
            cp = cc;
            hp = hc;
        };
        if (tp.ok && tp.pos0 + C <= L) {  // every position inside: no test per position
#pragma unroll
            for (int i = 0; i < C; ++i) {
                cell(i);
                acc = i == 0 ? e[0].m : MonoidT<2>::then(acc, e[i].m);
            }
            return acc;
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if (tp.ok && tp.pos0 + i < L) {
                cell(i);
            } else {
                e[i].m = MonoidT<2>::id();
                e[i].cc = 0.0f;
                e[i].hc = 0.0f;
            }
            acc = i == 0 ? e[0].m : MonoidT<2>::then(acc, e[i].m);
        }
        return acc;
    }

    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float2s d) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        uint32_t mx = 0;
        const auto update = [&](int i) {
            d = MonoidT<2>::apply(e[i].m, d);
            const float cn = e[i].cc + d.x;
            const float hn = e[i].hc + d.y;
            c[base + i * H] = cn;
            h[base + i * H] = hn;
            const uint32_t a0 = abs_bits(d.x), a1 = abs_bits(d.y);
            mx = a0 > mx ? a0 : mx;
            mx = a1 > mx ? a1 : mx;
            if (i == C - 1 && tp.sub == tp.nsub - 1)
                bnd_next[tp.q * B * H + tp.b * H + tp.j] = make_float2(cn, hn);
        };
        if (tp.ok && tp.pos0 + C <= L) {
#pragma unroll
            for (int i = 0; i < C; ++i) update(i);
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i)
                if (tp.ok && tp.pos0 + i < L) update(i);
        }
        wg_max_to<NW>(mx, maxd + (k - 1));
    }
};

// ---------------------------------------------------------------- finalize
// info = {first k with e_k <= tol, 1} or {cap, 0}; trace[k-1] = e_k.
__global__ void newton_finalize(const uint32_t *maxd, int cap, float tol, int32_t *info,
                                float *trace) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int it = cap, conv = 0;
    for (int k = 0; k < cap; ++k) {
        const float e = __uint_as_float(maxd[k]);
        if (trace) trace[k] = e;
        if (!conv && e <= tol) {
            it = k + 1;
            conv = 1;
        }
    }
    if (info) {
        info[0] = it;
        info[1] = conv;
    }
}

hipError_t newton_finalize_launch(const uint32_t *maxd, int cap, float tol, int32_t *info, float *trace,
                                  hipStream_t s) {
    hipLaunchKernelGGL(newton_finalize, dim3(1), dim3(64), 0, s, maxd, cap, tol, info, trace);
    return hipGetLastError();
}

// Warm start of the per-iteration path: the initial iterate (h, and c for
// S = 2; a null one is zero) copied into the outputs, and its state at the
// last position of every chunk into the boundary array iteration 1 reads.
struct SeedArgs {
    const float *h_init, *c_init;
    float *h, *c;
    void *bnd;
    int64_t B, L, H, T;
};

template <int S>
__global__ __launch_bounds__(256) void newton_seed_kernel(SeedArgs a) {
    const int64_t n = a.B * a.L * a.H;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = e % a.H, bt = e / a.H, t = bt % a.L, b = bt / a.L;
        const float hv = a.h_init != nullptr ? a.h_init[e] : 0.0f;
        a.h[e] = hv;
        float cv = 0.0f;
        if constexpr (S == 2) {
            cv = a.c_init != nullptr ? a.c_init[e] : 0.0f;
            a.c[e] = cv;
        }
        if ((t + 1) % a.T == 0 || t == a.L - 1) {
            const int64_t slot = (t / a.T) * a.B * a.H + b * a.H + j;
            if constexpr (S == 1)
                static_cast<float *>(a.bnd)[slot] = hv;
            else
                static_cast<float2 *>(a.bnd)[slot] = make_float2(cv, hv);
        }
    }
}

hipError_t newton_seed1(const float *init, float *h, float *bnd, int64_t B, int64_t L, int64_t H, int64_t T,
                        hipStream_t s) {
    SeedArgs a{init, nullptr, h, nullptr, bnd, B, L, H, T};
    const int64_t n = B * L * H;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, (int64_t)device_cu_count() * 8);
    hipLaunchKernelGGL(newton_seed_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Runs the launch sequence shared by both cells.  `make_op(k, bnd_prev,
// bnd_next, maxd)` returns the op of iteration k.  `seed`, when not null,
// holds a warm start's initial iterate (its bnd and T are set here).
template <int S, int NWC, int CC, int NWT, int CT, class MakeOp>
static hipError_t newton_loop(const TileCfg &cfg, int64_t B, int64_t L, int64_t H, int32_t cap,
                              float tol, int32_t *info, float *trace, const Ws &ws, hipStream_t s,
                              SeedArgs *seed, MakeOp make_op) {
    const NewtonWs w = newton_ws(cfg, S, B, L, H, cap);
    FillRange fr[1] = {{ws.p + w.maxd, (uint64_t)cap, 0, 4}};
    hipError_t e = fill(fr, 1, s);
    if (e != hipSuccess) return e;
    if (seed != nullptr) {
        seed->bnd = ws.p + w.bnd[0];  // iteration 1 reads bnd[0] as its previous iterate's
        seed->T = w.sh.T;
        const int64_t n = B * L * H;
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, (int64_t)device_cu_count() * 8);
        hipLaunchKernelGGL(newton_seed_kernel<S>, dim3((unsigned)blocks), dim3(256), 0, s, *seed);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    uint32_t *maxd = reinterpret_cast<uint32_t *>(ws.p + w.maxd);
    ScanGeo g;
    g.B = B;
    g.L = L;
    g.H = H;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.ws = ws_span(ws, w.maxd, w.keep_end);  // max|delta| slots and boundary states outlive a launch
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    for (int k = 1; k <= cap; ++k) {
        const int par = k & 1;
        auto op = make_op(k, ws.p + w.bnd[par ^ 1], ws.p + w.bnd[par], maxd);
        e = w.sh.channel_lanes ? launch_chunk_scan<decltype(op), NWC, CC, true>(op, g, s)
                               : launch_chunk_scan<decltype(op), NWT, CT, false>(op, g, s);
        if (e != hipSuccess) return e;
    }
    if (info != nullptr || trace != nullptr) {
        hipLaunchKernelGGL(newton_finalize, dim3(1), dim3(64), 0, s, maxd, cap, tol, info, trace);
        e = hipGetLastError();
    }
    return e;
}


hipError_t gru_forward_step(const GruFwdArgs &a, const Ws &ws, hipStream_t s) {
    auto make = [&](int k, char *bprev, char *bnext, uint32_t *maxd) {
        GruStepOp op;
        op.pz = a.pz;
        op.pr = a.pr;
        op.pc = a.pc;
        op.uz = a.uz;
        op.ur = a.ur;
        op.uc = a.uc;
        op.h0 = a.h0;
        op.h = a.h;
        op.bnd_prev = reinterpret_cast<const float *>(bprev);
        op.bnd_next = reinterpret_cast<float *>(bnext);
        op.maxd = maxd;
        op.tol = a.tol;
        op.k = k;
        op.cold1 = k == 1 && a.h_init == nullptr;
        op.B = a.B;
        op.L = a.L;
        op.H = a.H;
        op.runs = a.H == 1 && a.L % 4 == 0 && aligned16(a.pz) && aligned16(a.pr) && aligned16(a.pc) &&
                  aligned16(a.h);
        return op;
    };
    constexpr TileCfg c = kCfgGruStep;
    SeedArgs seed{a.h_init, nullptr, a.h, nullptr, nullptr, a.B, a.L, a.H, 0};
    return newton_loop<1, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl>(c, a.B, a.L, a.H, a.cap, a.tol, a.info, a.trace, ws, s,
                                                            a.h_init != nullptr ? &seed : nullptr, make);
}

hipError_t lstm_forward_step(const LstmFwdArgs &a, const Ws &ws, hipStream_t s) {
    auto make = [&](int k, char *bprev, char *bnext, uint32_t *maxd) {
        LstmStepOp op;
        op.pi = a.pi;
        op.pf = a.pf;
        op.po = a.po;
        op.pg = a.pg;
        op.ui = a.ui;
        op.uf = a.uf;
        op.uo = a.uo;
        op.ug = a.ug;
        op.h0 = a.h0;
        op.c0 = a.c0;
        op.h = a.h;
        op.c = a.c;
        op.bnd_prev = reinterpret_cast<const float2 *>(bprev);
        op.bnd_next = reinterpret_cast<float2 *>(bnext);
        op.maxd = maxd;
        op.tol = a.tol;
        op.k = k;
        op.cold1 = k == 1 && a.h_init == nullptr && a.c_init == nullptr;
        op.B = a.B;
        op.L = a.L;
        op.H = a.H;
        return op;
    };
    constexpr TileCfg c = kCfgLstmStep;
    const bool warm = a.h_init != nullptr || a.c_init != nullptr;
    SeedArgs seed{a.h_init, a.c_init, a.h, a.c, nullptr, a.B, a.L, a.H, 0};
    return newton_loop<2, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl>(c, a.B, a.L, a.H, a.cap, a.tol, a.info, a.trace, ws, s,
                                                            warm ? &seed : nullptr, make);
}

}  // namespace prn
