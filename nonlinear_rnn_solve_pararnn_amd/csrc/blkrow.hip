// blkrow.hip -- k x k block linear recurrence h_t = A_t h_{t-1} + b_t for
// k = 4 and 8 (ParaRNN page, Fig. 2 caption: block bi-diagonal systems;
// DEER summary page, limitations paragraph: dense Jacobians within heads of
// a few channels), on the lane-group scan of lanegroup.hpp: each block's
// rows on a group of k lanes.  A wave's loads of one position are 64/k
// consecutive k x k blocks, 2 KB of contiguous rows for k = 8 and 1 KB for
// k = 4, each row read by its own lane.
#include "lanegroup.hpp"

namespace prn {
namespace {

using namespace lg;

// VEC: A 16-byte aligned, so block rows move as 16-byte pieces.
template <int K_, bool VEC>
struct LinRowOp {
    static constexpr int K = K_;
    const float *A, *b, *h0;
    float *h;
    int64_t L, H;

    struct Elem {
        RowK<K> m;
    };
    __device__ bool active() const { return true; }

    // Row c of the map of block e: VEC reads the row as 16-byte pieces and
    // reorders them (the piece holding column c first), otherwise each entry
    // is read alone at its xor position.
    __device__ void load_row(int64_t e, int c, RowK<K> &r) const {
        const float *row = A + (e * K + c) * K;
        if constexpr (VEC) {
            if constexpr (K == 4) {
                const float4 x = reinterpret_cast<const float4 *>(row)[0];
                float v[4] = {x.x, x.y, x.z, x.w};
                xor_order4(v, c);
#pragma unroll
                for (int p = 0; p < 4; ++p) r.a[p] = v[p];
            } else {
                const int own = c >> 2;  // the piece holding column c
                const float4 x = reinterpret_cast<const float4 *>(row)[own];
                const float4 y = reinterpret_cast<const float4 *>(row)[own ^ 1];
                float v[4] = {x.x, x.y, x.z, x.w}, u[4] = {y.x, y.y, y.z, y.w};
                xor_order4(v, c);
                xor_order4(u, c);
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    r.a[p] = v[p];      // columns c ^ p, p < 4: the own piece
                    r.a[p + 4] = u[p];  // columns c ^ p, p >= 4: the other piece
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < K; ++p) r.a[p] = row[c ^ p];
        }
        r.b = ld_once(b + e * K + c);
    }

    template <int C>
    __device__ RowK<K> phase1(const Pos &p, Elem (&e)[C]) const {
        // Branch-free: a position past the end (or a missing head) reads
        // block 0 and takes the identity map in its place.
        const int64_t base = (p.b * L + p.pos0) * H + p.j;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const bool v = p.ok && p.pos0 + i < L;
            load_row(v ? base + i * H : 0, p.c, e[i].m);
#pragma unroll
            for (int k = 0; k < K; ++k) e[i].m.a[k] = v ? e[i].m.a[k] : (k == 0 ? 1.0f : 0.0f);
            e[i].m.b = v ? e[i].m.b : 0.0f;
        }
        RowK<K> m = e[0].m;
#pragma unroll
        for (int i = 1; i < C; ++i) m = row_then<K>(m, e[i].m);
        return m;
    }

    __device__ float init_state(const Pos &p) const {
        return h0 != nullptr ? h0[(p.b * H + p.j) * K + p.c] : 0.0f;
    }

    template <int C, int NW>
    __device__ void phase2(const Pos &p, Elem (&e)[C], float x) const {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x = row_apply<K>(e[i].m, x);
            if (p.ok && p.pos0 + i < L) h[((p.b * L + p.pos0 + i) * H + p.j) * K + p.c] = x;
        }
    }
};

template <int K, int NW, int C, int MINW>
hipError_t run_blkrow(int64_t B, int64_t L, int64_t H, const float *A, const float *b, const float *h0,
                      float *h, const Ws &ws, hipStream_t s) {
    const BlkRowWs w = blkrow_ws(K, B, L, H);
    Geo g;
    g.B = B;
    g.L = L;
    g.H = H;
    g.ncb = w.ncb;
    g.nq = w.nq;
    g.ntiles = w.ntiles;
    g.nrow = w.nrow;
    g.ws = {reinterpret_cast<uint64_t *>(ws.p), (uint64_t)(ws.bytes / 8), 0, 0};
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    if (aligned16(A)) return launch<LinRowOp<K, true>, NW, C, MINW>(LinRowOp<K, true>{A, b, h0, h, L, H}, g, s);
    return launch<LinRowOp<K, false>, NW, C, MINW>(LinRowOp<K, false>{A, b, h0, h, L, H}, g, s);
}

}  // namespace

hipError_t linscan_blkrow(int k, int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                          const float *h0, float *h, const Ws &ws, hipStream_t s) {
    if (k == 8) return run_blkrow<8, kBlkRow8.nw, kBlkRow8.c, kBlkRow8.minw>(B, L, H, A, b, h0, h, ws, s);
    if (k == 4) return run_blkrow<4, kBlkRow4.nw, kBlkRow4.c, kBlkRow4.minw>(B, L, H, A, b, h0, h, ws, s);
    return hipErrorInvalidValue;
}

}  // namespace prn
