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
#include "lanegroup.hpp"
#include "newton_iter.hpp"

namespace prn {
namespace {

using namespace lg;

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

    // Row c of one weight matrix of head j, in xor order.
    __device__ static void row(const float *U, const Pos &p, float (&u)[K]) {
        const float *r = U + (p.j * K + p.c) * K;
#pragma unroll
        for (int q = 0; q < K; ++q) u[q] = r[p.c ^ q];
    }

    // Newton map of one position: row c of the Jacobian at the previous state
    // hp (this lane's component; the others come from the group) and
    // beta = F - s.
    __device__ static void cell(float hp, float xz, float xr, float xc, const float (&uz)[K], const float (&ur)[K],
                                const float (&uc)[K], float s, RowK<K> &m) {
        float az = xz, ar = xr;
        xor_terms_sum<K>(hp, uz, az);
        xor_terms_sum<K>(hp, ur, ar);
        const float z = sigmoid(az), r = sigmoid(ar);
        float ac = xc;
        xor_terms_sum<K>(r * hp, uc, ac);
        const float cc = tanh_fast(ac);
        const float a1 = (cc - hp) * (z - z * z);
        const float a2 = z * fmaf(-cc, cc, 1.0f);
        float wx[K];
        xor_lanes<K>(hp * (r - r * r), wx);  // h_m r_m (1 - r_m) of lane c ^ q
        float vq[K], t[K], rx[K];
#pragma unroll
        for (int q = 0; q < K; ++q) {
            vq[q] = uc[q] * wx[q];
            t[q] = 0.0f;
            rx[q] = 0.0f;
        }
        ur_terms<0>(ur, vq, t);        // t[p] = sum_m Uc[c][m] w_m Ur[m][c ^ p]
        xor_terms<K, 0>(r, uc, rx);    // rx[p] = Uc[c][c ^ p] r_{c ^ p}
#pragma unroll
        for (int q = 0; q < K; ++q) m.a[q] = fmaf(a1, uz[q], a2 * (rx[q] + t[q])) + (q == 0 ? 1.0f - z : 0.0f);
        m.b = fmaf(z, cc - hp, hp) - s;
    }
    // t[q ^ M] += vq[q] * (lane c^q's ur[M]) for every M: lane c^q holds
    // Ur[c^q][c^q^M], so the sum over q is column c ^ p of (vq) Ur.
    template <int M>
    __device__ static void ur_terms(const float (&ur)[K], const float (&vq)[K], float (&t)[K]) {
        if constexpr (M < K) {
            xor_terms<K, M>(ur[M], vq, t);
            ur_terms<M + 1>(ur, vq, t);
        }
    }

    template <int C>
    __device__ RowK<K> phase1(const Pos &p, Elem (&e)[C]) const {
        float uz[K], ur[K], uc[K];
        if (p.ok) {
            row(Uz, p, uz);
            row(Ur, p, ur);
            row(Uc, p, uc);
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

}  // namespace

hipError_t hgru_forward(const HgruFwdArgs &a, const Ws &ws, hipStream_t s) {
    if (a.k == 8) return run_hgru<8, kHgru8.nw, kHgru8.c, kHgru8.minw>(a, ws, s);
    if (a.k == 4) return run_hgru<4, kHgru4.nw, kHgru4.c, kHgru4.minw>(a, ws, s);
    return hipErrorInvalidValue;
}

}  // namespace prn
