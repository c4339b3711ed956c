// hgru.hip -- Newton's method for the GRU with dense recurrence inside heads
// of k channels (k = 4, 8), whose Jacobian is block-diagonal with dense k x k
// blocks (DEER summary page, limitations paragraph: dense Jacobians, the GRU
// with heads of 8 channels; ParaRNN page, Fig. 2 caption: block bi-diagonal
// systems).  The cell is the diagonal GRU cell with each weight vector u
// replaced by one k x k matrix per head, acting on the state where u
// multiplies it (a diagonal U gives the diagonal cell):
//   z = s(pz + Uz h), r = s(pr + Ur h), c = tanh(pc + Uc (r h)),
//   F = h + z (c - h)
//   dF_i/dh_l = [i = l](1 - z_i) + (c_i - h_i) z_i (1 - z_i) Uz[i][l]
//             + z_i (1 - c_i^2) (Uc[i][l] r_l + sum_m Uc[i][m] h_m r_m (1 - r_m) Ur[m][l])
//
// One launch per Newton iteration, on the lane-group scan (lanegroup.hpp):
// lane c of a group of k lanes evaluates row c of the cell, and of its
// Jacobian in xor order, from the state vector of its head (exchanged by
// DPP) and row c of each weight matrix; the last sum is the product of the
// row-distributed Ur with the vector Uc[c][m] h_m r_m (1 - r_m), composed the
// way two maps are.  Iteration k (from s^0 = 0, or the caller's initial
// iterate) reads the gate inputs and s^{k-1} and writes s^k in place:
//   beta_t = F(s^{k-1}_{t-1}) - s^{k-1}_t,  delta_t = J_t delta_{t-1} + beta_t,
//   s^k = s^{k-1} + delta,  e_k = max |delta| (NaN counts as +inf).
// As on the per-iteration path of the diagonal cells (newton_step.hip), the
// last state of every chunk is also kept in a boundary array for the next
// launch, every launch first reads e_{k-1}, and launches after convergence
// exit at once.
//
// Gradients (DEER summary: forward plus gradients) come from the adjoint of
// the converged sequence, on the same lane-group scan in reverse time:
//   nu_t = J_t^T (nu_{t+1} + g_t),  nu_L = 0,  lambda_t = g_t + nu_{t+1},
// then, with a1 = dF/daz and a2 = dF/dac of each component and
// w = h r (1 - r) at the previous state,
//   dL/dpz = lambda a1,  dL/dpc = lambda a2 =: v,  dL/dpr = w (Uc^T v),
//   dL/dUz += (lambda a1) h^T,  dL/dUr += (dL/dpr) h^T,  dL/dUc += v (r h)^T,
//   dL/dh0 = nu_0.
// Lane c holds row c of J_t^T in xor order: entry p of lane c ^ p of the
// Jacobian row (xor_each), so the transpose costs one exchange per entry.
#include "lanegroup.hpp"
#include "newton_iter.hpp"

namespace prn {
namespace {

using namespace lg;

// Row c of one weight matrix of head j, in xor order: u[q] = U[j][c][c ^ q].
template <int K>
__device__ __forceinline__ void weight_row(const float *U, int64_t j, int c, float (&u)[K]) {
    const float *r = U + (j * K + c) * K;
#pragma unroll
    for (int q = 0; q < K; ++q) u[q] = r[c ^ q];
}

// t[q ^ M] += vq[q] * (lane c^q's ur[M]) for every M: lane c^q holds
// Ur[c^q][c^q^M], so the sum over q is column c ^ p of (vq) Ur.
template <int K, int M>
__device__ __forceinline__ void ur_terms(const float (&ur)[K], const float (&vq)[K], float (&t)[K]) {
    if constexpr (M < K) {
        xor_terms<K, M>(ur[M], vq, t);
        ur_terms<K, M + 1>(ur, vq, t);
    }
}

// The cell of component c at the previous state hp (this lane's component;
// the others come from the group): its gates, the partials a1 = dF/daz and
// a2 = dF/dac, and row c of the Jacobian in xor order.
template <int K>
struct HgruRow {
    float a[K];
    float z, r, cc, a1, a2;
};

template <int K>
__device__ __forceinline__ void hgru_row(float hp, float xz, float xr, float xc, const float (&uz)[K],
                                         const float (&ur)[K], const float (&uc)[K], HgruRow<K> &o) {
    float az = xz, ar = xr;
    xor_terms_sum<K>(hp, uz, az);
    xor_terms_sum<K>(hp, ur, ar);
    const float z = sigmoid(az), r = sigmoid(ar);
    float ac = xc;
    xor_terms_sum<K>(r * hp, uc, ac);
    const float cc = tanh_fast(ac);
    const float a1 = (cc - hp) * fmaf(-z, z, z);
    const float a2 = z * fmaf(-cc, cc, 1.0f);
    float wx[K];
    xor_lanes<K>(hp * fmaf(-r, r, r), wx);  // h_m r_m (1 - r_m) of lane c ^ q
    // The row accumulates in place: a1 Uz[c][c ^ p] (+ 1 - z at p = 0), then
    // the two Uc terms with a2 already folded into the row of Uc.
    float a2uc[K], vq[K];
#pragma unroll
    for (int q = 0; q < K; ++q) {
        a2uc[q] = a2 * uc[q];
        vq[q] = a2uc[q] * wx[q];
        o.a[q] = q == 0 ? fmaf(a1, uz[q], 1.0f - z) : a1 * uz[q];
    }
    ur_terms<K, 0>(ur, vq, o.a);    // += a2 sum_m Uc[c][m] w_m Ur[m][c ^ p]
    xor_terms<K, 0>(r, a2uc, o.a);  // += a2 Uc[c][c ^ p] r_{c ^ p}
    o.z = z;
    o.r = r;
    o.cc = cc;
    o.a1 = a1;
    o.a2 = a2;
}

template <int K_>
struct HgruStepOp {
    static constexpr int K = K_;
    const float *pz, *pr, *pc, *Uz, *Ur, *Uc, *h0;
    float *h;
    const float *bnd_prev;
    float *bnd_next;
    uint32_t *maxd;
    float tol;
    int k;       // iteration
    bool cold1;  // iteration 1 from s^0 = 0 (no initial iterate)
    int64_t L, NH, nrow, T;

    struct Elem {
        RowK<K> m;  // row c of J_t (xor order) and beta_t[c]
        float s;    // s^{k-1}_t[c]
    };
    __device__ bool active() const { return newton_active(maxd, k, tol); }
    __device__ float init_state(const Pos &) const { return 0.0f; }  // no delta enters the first chunk

    // Newton map of one position: row c of the Jacobian at the previous state
    // hp and beta = F - s.
    __device__ static void cell(float hp, float xz, float xr, float xc, const float (&uz)[K], const float (&ur)[K],
                                const float (&uc)[K], float s, RowK<K> &m) {
        HgruRow<K> o;
        hgru_row<K>(hp, xz, xr, xc, uz, ur, uc, o);
#pragma unroll
        for (int q = 0; q < K; ++q) m.a[q] = o.a[q];
        m.b = fmaf(o.z, o.cc - hp, hp) - s;
    }

    template <int C>
    __device__ RowK<K> phase1(const Pos &p, Elem (&e)[C]) const {
        float uz[K], ur[K], uc[K];
        if (p.ok) {
            weight_row<K>(Uz, p.j, p.c, uz);
            weight_row<K>(Ur, p.j, p.c, ur);
            weight_row<K>(Uc, p.j, p.c, uc);
        } else {
#pragma unroll
            for (int q = 0; q < K; ++q) uz[q] = ur[q] = uc[q] = 0.0f;
        }
        const int64_t slot = (p.b * NH + p.j) * K + p.c;
        float hp = 0.0f;  // s^{k-1} before this sub-chunk (h0 before the sequence)
        if (p.ok) {
            if (p.pos0 == 0)
                hp = h0 != nullptr ? h0[slot] : 0.0f;
            else if (cold1)
                hp = 0.0f;
            else if (p.w == 0)
                hp = bnd_prev[(p.q - 1) * nrow + slot];  // the previous chunk may be overwritten already
            else if (p.pos0 <= L)  // a sub-chunk wholly past the end reads nothing
                hp = h[((p.b * L + p.pos0 - 1) * NH + p.j) * K + p.c];
        }
        // Every position is evaluated, with no branch per position (the DPP
        // exchanges run on whole lane groups either way): a position past the
        // end of the sequence or a head past NH runs on zeros and its map is
        // replaced by the identity.  All of the sub-chunk's loads are issued
        // before the first cell (an index outside reads element 0, replaced
        // by a select), so their latencies overlap.
        float xs[C], xz[C], xr[C], xc[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t t = p.pos0 + i;
            const bool val = p.ok && t < L;  // uniform over the lane group
            const int64_t idx = ((p.b * L + (val ? t : 0)) * NH + (p.ok ? p.j : 0)) * K + p.c;
            xs[i] = cold1 ? 0.0f : h[idx];
            xz[i] = ld_once(pz + idx);
            xr[i] = ld_once(pr + idx);
            xc[i] = ld_once(pc + idx);
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const bool val = p.ok && p.pos0 + i < L;
            const float s = val ? xs[i] : 0.0f;
            RowK<K> m;
            cell(hp, val ? xz[i] : 0.0f, val ? xr[i] : 0.0f, val ? xc[i] : 0.0f, uz, ur, uc, s, m);
#pragma unroll
            for (int q = 0; q < K; ++q) e[i].m.a[q] = val ? m.a[q] : (q == 0 ? 1.0f : 0.0f);
            e[i].m.b = val ? m.b : 0.0f;
            e[i].s = s;
            hp = s;
        }
        RowK<K> acc = e[0].m;
#pragma unroll
        for (int i = 1; i < C; ++i) acc = row_then<K>(acc, e[i].m);
        return acc;
    }

    template <int C, int NW>
    __device__ void phase2(const Pos &p, Elem (&e)[C], float d) const {
        const int64_t slot = (p.b * NH + p.j) * K + p.c;
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            d = row_apply<K>(e[i].m, d);
            const int64_t t = p.pos0 + i;
            if (p.ok && t < L) {
                const float sn = e[i].s + d;
                h[((p.b * L + t) * NH + p.j) * K + p.c] = sn;
                const uint32_t ad = abs_bits(d);
                mx = ad > mx ? ad : mx;
                if (t == (p.q + 1) * T - 1) bnd_next[p.q * nrow + slot] = sn;  // the chunk's last state
            }
        }
        wg_max_to<NW>(mx, maxd + (k - 1));
    }
};

template <int K, int NW, int C, int MINW>
hipError_t run_hgru(const HgruFwdArgs &a, const Ws &ws, hipStream_t s) {
    const HgruWs w = hgru_ws(K, a.B, a.L, a.NH, a.cap);
    FillRange fr[1] = {{ws.p + w.maxd, (uint64_t)a.cap, 0, 4}};
    hipError_t e = fill(fr, 1, s);
    if (e != hipSuccess) return e;
    if (a.h_init != nullptr) {
        // iteration 1 reads bnd[0] as its previous iterate's chunk-end states
        e = newton_seed1(a.h_init, a.h, reinterpret_cast<float *>(ws.p + w.bnd[0]), a.B, a.L, a.NH * K, w.sh.T, s);
        if (e != hipSuccess) return e;
    }
    uint32_t *maxd = reinterpret_cast<uint32_t *>(ws.p + w.maxd);
    Geo g;
    g.B = a.B;
    g.L = a.L;
    g.H = a.NH;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.nrow = w.sh.nrow;
    // max|delta| slots and boundary states outlive a launch: kept at a wrap clear
    g.ws = {reinterpret_cast<uint64_t *>(ws.p), (uint64_t)(ws.bytes / 8), (uint64_t)(w.maxd / 8),
            (uint64_t)(w.keep_end / 8)};
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    for (int k = 1; k <= a.cap; ++k) {
        const int par = k & 1;
        HgruStepOp<K> op;
        op.pz = a.pz;
        op.pr = a.pr;
        op.pc = a.pc;
        op.Uz = a.Uz;
        op.Ur = a.Ur;
        op.Uc = a.Uc;
        op.h0 = a.h0;
        op.h = a.h;
        op.bnd_prev = reinterpret_cast<const float *>(ws.p + w.bnd[par ^ 1]);
        op.bnd_next = reinterpret_cast<float *>(ws.p + w.bnd[par]);
        op.maxd = maxd;
        op.tol = a.tol;
        op.k = k;
        op.cold1 = k == 1 && a.h_init == nullptr;
        op.L = a.L;
        op.NH = a.NH;
        op.nrow = w.sh.nrow;
        op.T = w.sh.T;
        e = launch<HgruStepOp<K>, NW, C, MINW>(op, g, s);
        if (e != hipSuccess) return e;
    }
    if (a.info != nullptr || a.trace != nullptr) e = newton_finalize_launch(maxd, a.cap, a.tol, a.info, a.trace, s);
    return e;
}

// ---------------------------------------------------------------- adjoint
// Position pos of the scan is time t = L - 1 - pos.  The map of position pos
// takes nu_{t+1} to nu_t: row c of J_t^T and (J_t^T g_t)[c].
template <int K_>
struct HgruAdjOp {
    static constexpr int K = K_;
    static constexpr int G = 64 / K;  // heads per wave
    const float *pz, *pr, *pc, *Uz, *Ur, *Uc, *h0, *h, *gh;
    float *gpz, *gpr, *gpc, *gh0;
    float *partial;  // [tile][G][3][K][K] rows of dL/dU per (tile, head), or null
    int64_t B, L, NH, ncb;

    struct Elem {
        RowK<K> m;
        float g, a1, a2, hp, r;  // g_t[c]; partials; previous state and reset gate of component c
    };
    __device__ bool active() const { return true; }
    __device__ float init_state(const Pos &) const { return 0.0f; }  // nu_L = 0

    template <int C>
    __device__ RowK<K> phase1(const Pos &p, Elem (&e)[C]) const {
        float uz[K], ur[K], uc[K];
        if (p.ok) {
            weight_row<K>(Uz, p.j, p.c, uz);
            weight_row<K>(Ur, p.j, p.c, ur);
            weight_row<K>(Uc, p.j, p.c, uc);
        } else {
#pragma unroll
            for (int q = 0; q < K; ++q) uz[q] = ur[q] = uc[q] = 0.0f;
        }
        const int64_t jj = p.ok ? p.j : 0;
        const float hinit = h0 != nullptr ? h0[(p.b * NH + jj) * K + p.c] : 0.0f;
        // every load of the sub-chunk first, none behind a branch (an index
        // outside the sequence reads time 0 and is replaced by a select)
        float xz[C], xr[C], xc[C], xg[C], xh[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t pos = p.pos0 + i;
            const bool val = p.ok && pos < L;  // uniform over the lane group
            const int64_t t = val ? L - 1 - pos : 0;
            const int64_t idx = ((p.b * L + t) * NH + jj) * K + p.c;
            xz[i] = ld_once(pz + idx);
            xr[i] = ld_once(pr + idx);
            xc[i] = ld_once(pc + idx);
            xg[i] = ld_once(gh + idx);
            const float hv = h[t > 0 ? idx - NH * K : idx];
            xh[i] = t > 0 ? hv : hinit;
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const bool val = p.ok && p.pos0 + i < L;
            HgruRow<K> o;
            hgru_row<K>(xh[i], xz[i], xr[i], xc[i], uz, ur, uc, o);
            float at[K];
            xor_each<K>(o.a, at);  // row c of J_t^T
            float bt = 0.0f;
            xor_terms_sum<K>(xg[i], at, bt);  // (J_t^T g_t)[c]
#pragma unroll
            for (int q = 0; q < K; ++q) e[i].m.a[q] = val ? at[q] : (q == 0 ? 1.0f : 0.0f);
            e[i].m.b = val ? bt : 0.0f;
            e[i].g = val ? xg[i] : 0.0f;
            e[i].a1 = val ? o.a1 : 0.0f;
            e[i].a2 = val ? o.a2 : 0.0f;
            e[i].hp = xh[i];
            e[i].r = o.r;
        }
        RowK<K> acc = e[0].m;
#pragma unroll
        for (int i = 1; i < C; ++i) acc = row_then<K>(acc, e[i].m);
        return acc;
    }

    template <int C, int NW>
    __device__ void phase2(const Pos &p, Elem (&e)[C], float x) const {
        float uct[K];  // row c of Uc^T, xor order
        {
            float uc[K];
            if (p.ok) {
                weight_row<K>(Uc, p.j, p.c, uc);
            } else {
#pragma unroll
                for (int q = 0; q < K; ++q) uc[q] = 0.0f;
            }
            xor_each<K>(uc, uct);
        }
        const bool want_u = partial != nullptr;
        float dz[K], dr[K], dc[K];
#pragma unroll
        for (int q = 0; q < K; ++q) dz[q] = dr[q] = dc[q] = 0.0f;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int64_t pos = p.pos0 + i;
            const bool val = p.ok && pos < L;
            const float lam = e[i].g + x;  // lambda_t = g_t + nu_{t+1}
            x = row_apply<K>(e[i].m, x);   // nu_t
            const float vz = lam * e[i].a1, vc = lam * e[i].a2;
            float q = 0.0f;
            xor_terms_sum<K>(vc, uct, q);  // (Uc^T v)[c]
            const float vr = q * (e[i].hp * (e[i].r - e[i].r * e[i].r));
            if (val) {
                const int64_t t = L - 1 - pos;
                const int64_t idx = ((p.b * L + t) * NH + p.j) * K + p.c;
                gpz[idx] = vz;
                gpr[idx] = vr;
                gpc[idx] = vc;
                if (t == 0 && gh0 != nullptr) gh0[(p.b * NH + p.j) * K + p.c] = x;
            }
            if (want_u) {  // uniform over the launch
                float xh[K], xrh[K];
                xor_lanes<K>(e[i].hp, xh);
                xor_lanes<K>(e[i].r * e[i].hp, xrh);
#pragma unroll
                for (int m = 0; m < K; ++m) {
                    dz[m] = fmaf(vz, xh[m], dz[m]);
                    dr[m] = fmaf(vr, xh[m], dr[m]);
                    dc[m] = fmaf(vc, xrh[m], dc[m]);
                }
            }
        }
        if (!want_u) return;
        // sum over the waves (the workgroup's sub-chunks of the same heads),
        // then one partial per (tile, head); the next tile writes s_red only
        // after the ticket barrier, which wave 0 passes after its reads
        __shared__ float s_red[NW][3 * K][64];
#pragma unroll
        for (int m = 0; m < K; ++m) {
            s_red[p.w][m][p.lane] = dz[m];
            s_red[p.w][K + m][p.lane] = dr[m];
            s_red[p.w][2 * K + m][p.lane] = dc[m];
        }
        __syncthreads();
        if (p.w == 0) {
            const int64_t tile = (p.q * B + p.b) * ncb + p.j / G;
            float *out = partial + (tile * G + p.lane / K) * (3 * K * K);
#pragma unroll
            for (int gate = 0; gate < 3; ++gate) {
#pragma unroll
                for (int m = 0; m < K; ++m) {
                    float v = 0.0f;
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) v += s_red[ww][gate * K + m][p.lane];
                    out[gate * K * K + p.c * K + (p.c ^ m)] = v;  // row c, column c ^ m
                }
            }
        }
    }
};

// dL/dU: the per-tile partials of each head summed over chunks and batch
// rows in two fixed-order passes.  Pass 1: block (head j, gate, slice) sums
// the tiles m = q * B + b of its slice (kHgruUSlices slices) into stage;
// pass 2: block (head j, gate) sums the slices.  Pass 1 has enough blocks to
// keep every CU reading.
struct HgruUReduce {
    const float *partial;
    float *stage;  // [NH][3][kHgruUSlices][k * k]
    float *gu[3];
    int64_t B, nq, ncb;
    int k;
};

__global__ __launch_bounds__(256) void hgru_u_slice_kernel(HgruUReduce r) {
    __shared__ float red[256];
    const int64_t j = blockIdx.x;
    const int gate = blockIdx.y, slice = blockIdx.z;
    if (r.gu[gate] == nullptr) return;
    const int kk = r.k * r.k, heads = 64 / r.k;
    const int e = threadIdx.x % kk, part = threadIdx.x / kk, nparts = 256 / kk;
    const int64_t cb = j / heads, g = j % heads, n = r.nq * r.B;
    const int64_t per = (n + kHgruUSlices - 1) / kHgruUSlices;
    const int64_t lo = slice * per, hi = lo + per < n ? lo + per : n;
    float s = 0.0f;
    for (int64_t m = lo + part; m < hi; m += nparts) {  // m = q * B + b
        const int64_t tile = m * r.ncb + cb;
        s += r.partial[((tile * heads + g) * 3 + gate) * kk + e];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    if ((int)threadIdx.x < kk) {
        float t = 0.0f;
        for (int q = 0; q < nparts; ++q) t += red[q * kk + threadIdx.x];
        r.stage[((j * 3 + gate) * kHgruUSlices + slice) * kk + threadIdx.x] = t;
    }
}

__global__ __launch_bounds__(64) void hgru_u_sum_kernel(HgruUReduce r) {
    const int64_t j = blockIdx.x;
    const int gate = blockIdx.y;
    float *out = r.gu[gate];
    const int kk = r.k * r.k;
    if (out == nullptr || (int)threadIdx.x >= kk) return;
    float t = 0.0f;
    for (int q = 0; q < kHgruUSlices; ++q) t += r.stage[((j * 3 + gate) * kHgruUSlices + q) * kk + threadIdx.x];
    out[j * kk + threadIdx.x] = t;
}

template <int K, int NW, int C, int MINW>
hipError_t run_hgru_adj(const HgruBwdArgs &a, const Ws &ws, hipStream_t s) {
    const HgruAdjWs w = hgru_adj_ws(K, a.B, a.L, a.NH);
    const bool want_u = a.gU[0] != nullptr || a.gU[1] != nullptr || a.gU[2] != nullptr;
    HgruAdjOp<K> op;
    op.pz = a.pz;
    op.pr = a.pr;
    op.pc = a.pc;
    op.Uz = a.Uz;
    op.Ur = a.Ur;
    op.Uc = a.Uc;
    op.h0 = a.h0;
    op.h = a.h;
    op.gh = a.gh;
    op.gpz = a.gpz;
    op.gpr = a.gpr;
    op.gpc = a.gpc;
    op.gh0 = a.gh0;
    op.partial = want_u ? reinterpret_cast<float *>(ws.p + w.partial) : nullptr;
    op.B = a.B;
    op.L = a.L;
    op.NH = a.NH;
    op.ncb = w.sh.ncb;
    Geo g;
    g.B = a.B;
    g.L = a.L;
    g.H = a.NH;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.nrow = w.sh.nrow;
    // the partials are read by the next launch: kept at a wrap clear
    g.ws = {reinterpret_cast<uint64_t *>(ws.p), (uint64_t)(ws.bytes / 8), (uint64_t)(w.partial / 8),
            (uint64_t)(w.total / 8)};
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.sh.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.sh.inc);
    hipError_t e = launch<HgruAdjOp<K>, NW, C, MINW>(op, g, s);
    if (e != hipSuccess || !want_u) return e;
    HgruUReduce r;
    r.partial = op.partial;
    r.stage = reinterpret_cast<float *>(ws.p + w.stage);
    for (int q = 0; q < 3; ++q) r.gu[q] = a.gU[q];
    r.B = a.B;
    r.nq = w.sh.nq;
    r.ncb = w.sh.ncb;
    r.k = K;
    hipLaunchKernelGGL(hgru_u_slice_kernel, dim3((unsigned)a.NH, 3, kHgruUSlices), dim3(256), 0, s, r);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(hgru_u_sum_kernel, dim3((unsigned)a.NH, 3), dim3(64), 0, s, r);
    return hipGetLastError();
}

}  // namespace

hipError_t hgru_forward(const HgruFwdArgs &a, const Ws &ws, hipStream_t s) {
    if (a.k == 8) return run_hgru<8, kHgru8.nw, kHgru8.c, kHgru8.minw>(a, ws, s);
    if (a.k == 4) return run_hgru<4, kHgru4.nw, kHgru4.c, kHgru4.minw>(a, ws, s);
    return hipErrorInvalidValue;
}

hipError_t hgru_backward(const HgruBwdArgs &a, const Ws &ws, hipStream_t s) {
    if (a.k == 8) return run_hgru_adj<8, kHgruAdj8.nw, kHgruAdj8.c, kHgruAdj8.minw>(a, ws, s);
    if (a.k == 4) return run_hgru_adj<4, kHgruAdj4.nw, kHgruAdj4.c, kHgruAdj4.minw>(a, ws, s);
    return hipErrorInvalidValue;
}

}  // namespace prn
