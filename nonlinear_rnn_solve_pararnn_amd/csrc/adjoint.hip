// adjoint.hip -- gradients through the converged sequence by a reverse-time
// linear scan (DEER summary: forward plus gradients).
//
// For L = sum_t g_t . s_t the adjoint obeys
//   lambda_t = g_t + J_{t+1}^T lambda_{t+1},
// whose coefficient J_{t+1} belongs to the next position.  Writing
// nu_t = J_t^T lambda_t turns it into a recurrence with position-local terms,
//   nu_t = J_t^T nu_{t+1} + J_t^T g_t,   lambda_t = g_t + nu_{t+1},
// an affine map per position scanned from t = L-1 down to 0 (nu_L = 0).
// Then dL/dp_t = (dF_t/dp_t)^T lambda_t, dL/du = sum_{b,t} of dL/dp_t times
// the derivative of the pre-activation by u, and dL/ds0 = nu_0.
// The scan core runs in "position" order; position pos is time L-1-pos.
#include "cells.hpp"
#include "launch.hpp"
#include "scan_core.hpp"

namespace prn {

// Sum of per-workgroup partials of dL/du over chunks and batch rows.
// partial layout: channel lanes [tile][gate][64]; time lanes [tile][gate].
struct UReduceArgs {
    const float *partial;
    float *gu[4];
    int ngates;
    int64_t B, H, nq, ncb;
    bool channel_lanes;
};

__global__ __launch_bounds__(256) void reduce_u_kernel(UReduceArgs r) {
    __shared__ float red[256];
    const int gate = blockIdx.y;
    const int64_t j = blockIdx.x;
    float *out = r.gu[gate];
    if (out == nullptr) return;
    const int64_t n = r.nq * r.B;
    float s = 0.0f;
    for (int64_t k = threadIdx.x; k < n; k += 256) {
        // k = q * B + b
        int64_t idx;
        if (r.channel_lanes)
            idx = ((k * r.ncb + j / 64) * r.ngates + gate) * 64 + (j % 64);
        else
            idx = (k * r.H + j) * r.ngates + gate;
        s += r.partial[idx];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int d = 128; d > 0; d >>= 1) {
        if ((int)threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[j] = red[0];
}

// Store per-workgroup dL/du partials of NG gates: every gate's per-thread sum
// is reduced over the workgroup to one value per channel lane (channel lanes:
// over the waves of each lane; time lanes: over every thread) in one pass,
// with a single barrier.  `red` is written again only by the next tile, whose
// workgroup has passed the ticket barrier (after wave 0's reads) by then.
template <int NW, bool CL, int NG>
__device__ __forceinline__ void store_u_partials(const TilePos &tp, const float (&su)[NG],
                                                 float *partial) {
    constexpr int W = CL ? NW * 64 : NW;  // slots per gate
    __shared__ float red[NG * W];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        if (CL) {
            red[q * W + w * 64 + lane] = su[q];
        } else {
            const float v = wave_sum(su[q]);
            if (lane == 0) red[q * W + w] = v;
        }
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            float s = 0.0f;
            for (int k = 0; k < NW; ++k) s += red[q * W + (CL ? k * 64 + lane : k)];
            if (CL)
                partial[(tp.tile * NG + q) * 64 + lane] = s;
            else if (lane == 0)
                partial[tp.tile * NG + q] = s;
        }
    }
}

// ---------------------------------------------------------------- GRU
struct GruAdjOp {
    static constexpr int S = 1;
    const float *pz, *pr, *pc, *uz, *ur, *uc, *h0, *h, *gh;
    float *gpz, *gpr, *gpc, *gh0;
    float *partial;  // NULL when no dL/du is wanted
    int64_t L, H;
    bool runs;  // H == 1 with 16-byte aligned rows: whole runs move as float4

    struct Elem {
        float J, g, dz, dr, dc, xz, xr, xc;  // xz.. = pre-activation derivative by u times dF/dp
    };
    __device__ bool active() const { return true; }
    __device__ float init_state(const TilePos &) const { return 0.0f; }

    // The C positions of a thread are the times tlo + C-1 down to tlo; as a
    // run in memory, position pos0 + i is element C-1-i.
    __device__ bool whole_run(const TilePos &tp, int C) const {
        return runs && tp.ok && tp.pos0 + C <= L;
    }

    template <int C>
    __device__ Aff1 phase1(const TilePos &tp, Elem (&e)[C]) const {
        const float wz = tp.ok ? uz[tp.j] : 0.0f, wr = tp.ok ? ur[tp.j] : 0.0f,
                    wc = tp.ok ? uc[tp.j] : 0.0f;
        Aff1 acc = {1.0f, 0.0f};
        if constexpr (C % 4 == 0) {
            if (whole_run(tp, C)) {
                const int64_t tlo = L - tp.pos0 - C;
                const int64_t blo = idx3(tp.b, tlo, tp.j, L, H);
                float vz[C], vr[C], vc[C], vg[C], vh[C];
                load_run<C, true>(pz + blo, vz);
                load_run<C, true>(pr + blo, vr);
                load_run<C, true>(pc + blo, vc);
                load_run<C, true>(gh + blo, vg);
                load_run<C>(h + blo, vh);
                const float hlo = tlo == 0 ? (h0 != nullptr ? h0[tp.b * H + tp.j] : 0.0f) : h[blo - 1];
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int m = C - 1 - i;
                    const float hp = m == 0 ? hlo : vh[m - 1];
                    float J, dz, dr, dc, r;
                    gru_j_dp(hp, vz[m], vr[m], vc[m], wz, wr, wc, J, dz, dr, dc, r);
                    e[i] = {J, vg[m], dz, dr, dc, dz * hp, dr * hp, dc * r * hp};
                    acc = {acc.a * J, fmaf(J, acc.b, J * vg[m])};
                }
                return acc;
            }
        }
        const auto cell = [&](int i) {
            const int64_t t = L - 1 - (tp.pos0 + i);
            const int64_t kk = idx3(tp.b, t, tp.j, L, H);
            const float hp = t == 0 ? (h0 != nullptr ? h0[tp.b * H + tp.j] : 0.0f) : h[kk - H];
            float J, dz, dr, dc, r;
            gru_j_dp(hp, ld_once(pz + kk), ld_once(pr + kk), ld_once(pc + kk), wz, wr, wc, J, dz, dr, dc, r);
            e[i] = {J, ld_once(gh + kk), dz, dr, dc, dz * hp, dr * hp, dc * r * hp};
        };
        if (tp.ok && tp.pos0 + C <= L) {  // every position inside: no test per position
#pragma unroll
            for (int i = 0; i < C; ++i) {
                cell(i);
                acc = {acc.a * e[i].J, fmaf(e[i].J, acc.b, e[i].J * e[i].g)};
            }
            return acc;
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if (tp.ok && tp.pos0 + i < L)
                cell(i);
            else
                e[i] = {1.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            acc = {acc.a * e[i].J, fmaf(e[i].J, acc.b, e[i].J * e[i].g)};
        }
        return acc;
    }

    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float nu) const {
        float su[3] = {0.0f, 0.0f, 0.0f};
        bool done = false;  // store_u_partials below must be reached by every thread
        if constexpr (C % 4 == 0) {
            if (whole_run(tp, C)) {
                const int64_t tlo = L - tp.pos0 - C;
                const int64_t blo = idx3(tp.b, tlo, tp.j, L, H);
                float oz[C], orr[C], oc[C];
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int m = C - 1 - i;
                    const float lam = e[i].g + nu;
                    oz[m] = e[i].dz * lam;
                    orr[m] = e[i].dr * lam;
                    oc[m] = e[i].dc * lam;
                    su[0] = fmaf(e[i].xz, lam, su[0]);
                    su[1] = fmaf(e[i].xr, lam, su[1]);
                    su[2] = fmaf(e[i].xc, lam, su[2]);
                    nu = e[i].J * lam;
                }
                store_run<C>(gpz + blo, oz);
                store_run<C>(gpr + blo, orr);
                store_run<C>(gpc + blo, oc);
                if (tlo == 0 && gh0 != nullptr) gh0[tp.b * H + tp.j] = nu;
                done = true;
            }
        }
        const auto update = [&](int i) {
            const int64_t t = L - 1 - (tp.pos0 + i);
            const int64_t kk = idx3(tp.b, t, tp.j, L, H);
            const float lam = e[i].g + nu;
            gpz[kk] = e[i].dz * lam;
            gpr[kk] = e[i].dr * lam;
            gpc[kk] = e[i].dc * lam;
            su[0] = fmaf(e[i].xz, lam, su[0]);
            su[1] = fmaf(e[i].xr, lam, su[1]);
            su[2] = fmaf(e[i].xc, lam, su[2]);
            nu = e[i].J * lam;
            if (t == 0 && gh0 != nullptr) gh0[tp.b * H + tp.j] = nu;
        };
        if (!done && tp.ok && tp.pos0 + C <= L) {
#pragma unroll
            for (int i = 0; i < C; ++i) update(i);
        } else if (!done) {
#pragma unroll
            for (int i = 0; i < C; ++i)
                if (tp.ok && tp.pos0 + i < L) update(i);
        }
        if (partial != nullptr) store_u_partials<NW, CL, 3>(tp, su, partial);
    }
};

// ---------------------------------------------------------------- LSTM
// State order (c, h) as (x, y).  Map nu -> J^T (g + nu).
//
// Per position only ten values are kept between the two phases; the rest of
// the Jacobian and of dh/dp follow from them (cells.hpp, LSTM partials):
//   j10 = odtc j00, j11 = uo dho + odtc j01, dh/dp_{i,f,g} = odtc dc/dp_{i,f,g},
// with odtc = o (1 - tanh^2 c) and dho = o (1 - o) tanh c.
struct LstmAdjOp {
    static constexpr int S = 2;
    const float *pi, *pf, *po, *pg, *ui, *uf, *uo, *ug, *h0, *c0, *h, *c, *gh, *gc;
    float *gpi, *gpf, *gpo, *gpg, *gh0, *gc0;
    float *partial;
    int64_t L, H;

    struct Elem {
        float j00, j01, gcv, ghv, dci, dcf, dcg, odtc, dho, hp;
    };
    __device__ bool active() const { return true; }
    __device__ float2s init_state(const TilePos &) const { return {0.0f, 0.0f}; }

    // Record and transposed map of position t (kk its element index).
    __device__ __forceinline__ Aff2 elem_at(const TilePos &tp, int64_t t, int64_t kk, float wi, float wf,
                                            float wo, float wg, Elem &e) const {
        float hp, cp;
        if (t == 0) {
            hp = h0 != nullptr ? h0[tp.b * H + tp.j] : 0.0f;
            cp = c0 != nullptr ? c0[tp.b * H + tp.j] : 0.0f;
        } else {
            hp = h[kk - H];
            cp = c[kk - H];
        }
        const LstmAdj r = lstm_adj(cp, hp, ld_once(pi + kk), ld_once(pf + kk), ld_once(po + kk),
                                   ld_once(pg + kk), wi, wf, wo, wg);
        e = {r.j00, r.j01, gc != nullptr ? ld_once(gc + kk) : 0.0f, ld_once(gh + kk),
             r.dci, r.dcf, r.dcg, r.odtc, r.dho, hp};
        // J^T and J^T g, with the two derived entries formed as phase2 forms them
        const float j10 = e.odtc * e.j00, j11 = fmaf(wo, e.dho, e.odtc * e.j01);
        return {e.j00, j10, e.j01, j11, fmaf(e.j00, e.gcv, j10 * e.ghv), fmaf(e.j01, e.gcv, j11 * e.ghv)};
    }

    template <int C>
    __device__ Aff2 phase1(const TilePos &tp, Elem (&e)[C]) const {
        float wi = 0.0f, wf = 0.0f, wo = 0.0f, wg = 0.0f;
        if (tp.ok) {
            wi = ui[tp.j];
            wf = uf[tp.j];
            wo = uo[tp.j];
            wg = ug[tp.j];
        }
        Aff2 acc;
        if (tp.ok && tp.pos0 + C <= L) {  // every position inside: no test per position
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const int64_t t = L - 1 - (tp.pos0 + i);
                const Aff2 m = elem_at(tp, t, idx3(tp.b, t, tp.j, L, H), wi, wf, wo, wg, e[i]);
                acc = i == 0 ? m : MonoidT<2>::then(acc, m);
            }
            return acc;
        }
        acc = MonoidT<2>::id();
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t pos = tp.pos0 + i;
            Aff2 m = MonoidT<2>::id();
            e[i] = {1.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            if (tp.ok && pos < L) {
                const int64_t t = L - 1 - pos;
                m = elem_at(tp, t, idx3(tp.b, t, tp.j, L, H), wi, wf, wo, wg, e[i]);
            }
            acc = MonoidT<2>::then(acc, m);
        }
        return acc;
    }

    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float2s nu) const {
        float su[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const float wo = tp.ok ? uo[tp.j] : 0.0f;
        const bool whole = tp.ok && tp.pos0 + C <= L;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t pos = tp.pos0 + i;
            if (whole || (tp.ok && pos < L)) {
                const int64_t t = L - 1 - pos;
                const int64_t kk = idx3(tp.b, t, tp.j, L, H);
                const float lc = e[i].gcv + nu.x, lh = e[i].ghv + nu.y;
                const float olh = e[i].odtc * lh;
                const float di = e[i].dci * (lc + olh);
                const float df = e[i].dcf * (lc + olh);
                const float dO = e[i].dho * lh;
                const float dg = e[i].dcg * (lc + olh);
                gpi[kk] = di;
                gpf[kk] = df;
                gpo[kk] = dO;
                gpg[kk] = dg;
                su[0] = fmaf(di, e[i].hp, su[0]);
                su[1] = fmaf(df, e[i].hp, su[1]);
                su[2] = fmaf(dO, e[i].hp, su[2]);
                su[3] = fmaf(dg, e[i].hp, su[3]);
                // nu = J^T lambda with j10 = odtc j00 and j11 = uo dho + odtc j01
                const float j10 = e[i].odtc * e[i].j00, j11 = fmaf(wo, e[i].dho, e[i].odtc * e[i].j01);
                nu = {fmaf(e[i].j00, lc, j10 * lh), fmaf(e[i].j01, lc, j11 * lh)};
                if (t == 0) {
                    if (gh0 != nullptr) gh0[tp.b * H + tp.j] = nu.y;
                    if (gc0 != nullptr) gc0[tp.b * H + tp.j] = nu.x;
                }
            }
        }
        if (partial != nullptr) store_u_partials<NW, CL, 4>(tp, su, partial);
    }
};

// ---------------------------------------------------------------- launch

size_t gru_adjoint_ws(int64_t B, int64_t L, int64_t H) {
    const ScanShape sh = scan_shape(kCfgGruAdj, B, L, H);
    return scan_ws(kCfgGruAdj, 1, B, L, H, (sh.channel_lanes ? 64 : 1) * 3).total;
}
size_t lstm_adjoint_ws(int64_t B, int64_t L, int64_t H) {
    const ScanShape sh = scan_shape(kCfgLstmAdj, B, L, H);
    return scan_ws(kCfgLstmAdj, 2, B, L, H, (sh.channel_lanes ? 64 : 1) * 4).total;
}

template <class Op, int S, int NWC, int CC, int NWT, int CT>
static hipError_t run_adjoint(const TileCfg &cfg, Op op, int ngates, const AdjArgs &a, const Ws &ws,
                              hipStream_t s) {
    const ScanShape sh0 = scan_shape(cfg, a.B, a.L, a.H);
    const ScanWs w = scan_ws(cfg, S, a.B, a.L, a.H, (sh0.channel_lanes ? 64 : 1) * ngates);
    bool want_u = false;
    for (int q = 0; q < ngates; ++q) want_u = want_u || a.gu[q] != nullptr;
    op.partial = want_u ? reinterpret_cast<float *>(ws.p + w.partial) : nullptr;
    ScanGeo g;
    g.B = a.B;
    g.L = a.L;
    g.H = a.H;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.ws = ws_span(ws, w.partial, w.keep_end);  // the dL/du partials are reduced by the next launch
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    hipError_t e = w.sh.channel_lanes ? launch_chunk_scan<Op, NWC, CC, true>(op, g, s)
                                      : launch_chunk_scan<Op, NWT, CT, false>(op, g, s);
    if (e != hipSuccess || !want_u) return e;
    UReduceArgs r;
    r.partial = op.partial;
    for (int q = 0; q < 4; ++q) r.gu[q] = q < ngates ? a.gu[q] : nullptr;
    r.ngates = ngates;
    r.B = a.B;
    r.H = a.H;
    r.nq = w.sh.nq;
    r.ncb = w.sh.ncb;
    r.channel_lanes = w.sh.channel_lanes;
    hipLaunchKernelGGL(reduce_u_kernel, dim3((unsigned)a.H, (unsigned)ngates), dim3(256), 0, s, r);
    return hipGetLastError();
}

hipError_t gru_adjoint(const AdjArgs &a, const Ws &ws, hipStream_t s) {
    GruAdjOp op;
    op.pz = a.p[0];
    op.pr = a.p[1];
    op.pc = a.p[2];
    op.uz = a.u[0];
    op.ur = a.u[1];
    op.uc = a.u[2];
    op.h0 = a.h0;
    op.h = a.h;
    op.gh = a.gh;
    op.gpz = a.gp[0];
    op.gpr = a.gp[1];
    op.gpc = a.gp[2];
    op.gh0 = a.gh0;
    op.partial = nullptr;
    op.L = a.L;
    op.H = a.H;
    op.runs = a.H == 1 && a.L % 4 == 0 && aligned16(a.p[0]) && aligned16(a.p[1]) && aligned16(a.p[2]) &&
              aligned16(a.h) && aligned16(a.gh) && aligned16(a.gp[0]) && aligned16(a.gp[1]) &&
              aligned16(a.gp[2]);
    constexpr TileCfg c = kCfgGruAdj;
    return run_adjoint<GruAdjOp, 1, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl>(c, op, 3, a, ws, s);
}

hipError_t lstm_adjoint(const AdjArgs &a, const Ws &ws, hipStream_t s) {
    LstmAdjOp op;
    op.pi = a.p[0];
    op.pf = a.p[1];
    op.po = a.p[2];
    op.pg = a.p[3];
    op.ui = a.u[0];
    op.uf = a.u[1];
    op.uo = a.u[2];
    op.ug = a.u[3];
    op.h0 = a.h0;
    op.c0 = a.c0;
    op.h = a.h;
    op.c = a.c;
    op.gh = a.gh;
    op.gc = a.gc;
    op.gpi = a.gp[0];
    op.gpf = a.gp[1];
    op.gpo = a.gp[2];
    op.gpg = a.gp[3];
    op.gh0 = a.gh0;
    op.gc0 = a.gc0;
    op.partial = nullptr;
    op.L = a.L;
    op.H = a.H;
    constexpr TileCfg c = kCfgLstmAdj;
    return run_adjoint<LstmAdjOp, 2, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl>(c, op, 4, a, ws, s);
}

}  // namespace prn
