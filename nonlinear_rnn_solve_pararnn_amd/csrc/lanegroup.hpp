// lanegroup.hpp -- chunked scans whose k x k maps are spread over a group of
// k lanes (k = 4, 8), and the single-pass scan tile that chains them: the
// machinery of the k x k block scans (rnn_linscan_blk) and of the Newton
// step of the cell with dense recurrence inside heads of k channels (ParaRNN
// page, Fig. 2 caption: block bi-diagonal systems; DEER summary page,
// limitations paragraph: dense Jacobians within heads of a few channels).
//
// A thread that held a whole 8x8 map would need 72 floats for the map it
// accumulates, 72 for each position it keeps for the second pass and more
// for the look-back: far past the register file.  Here lane c of a group of
// k lanes holds row c of every map of its block, with the row's entries in
// xor order,
//     a[p] = A[c][c ^ p]  (p = 0..k-1),   b = b[c],
// and component c of every state.  Composing two maps and applying a map to
// a state then need, from lane c, only the values of lanes c ^ p of the same
// group, which DPP moves inside a quad (xor 1, 2, 3) and inside a half row of
// 8 lanes (xor 7); nothing is indexed by lane in registers:
//     (A2 A1)[c][c ^ p'] = sum_p A2[c][c ^ p] * (lane c^p's a1[p ^ p'])
//     (A2 b1 + b2)[c]    = sum_p A2[c][c ^ p] * (lane c^p's b1) + b2[c]
//     (A x + b)[c]       = sum_p A[c][c ^ p]  * (lane c^p's x) + b[c]
// A wave holds 64/k blocks (heads) side by side.
//
// The scan is the same as for the other recurrences (scan_core.hpp): each
// lane runs serially over C positions and composes their maps, the NW waves
// of a workgroup (consecutive sub-chunks of the same heads) combine in LDS,
// and chunks are chained by a decoupled look-back over tagged records, one
// per (chunk, batch row, head, row).  Every decision of the look-back is
// taken for a whole lane group at once (a group folds a predecessor only
// when all k of its rows are published), since the DPP exchanges need the k
// lanes of a group to run together.  The per-position work comes from an Op:
// phase1 loads a sub-chunk and returns its composed map, phase2 receives the
// state component entering it and finishes it.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace prn {
namespace lg {

constexpr int kQpXor1 = 0xB1;       // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQpXor2 = 0x4E;       // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kQpXor3 = 0x1B;       // quad_perm [3,2,1,0]: lane ^ 3
constexpr int kHalfRowMirror = 0x141;  // lane i of 8 reads lane 7 - i: lane ^ 7

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// o[p] = v of lane (lane ^ p), p = 0..K-1
template <int K>
__device__ __forceinline__ void xor_lanes(float v, float (&o)[K]) {
    o[0] = v;
    o[1] = dpp_f<kQpXor1>(v);
    o[2] = dpp_f<kQpXor2>(v);
    o[3] = dpp_f<kQpXor3>(v);
    if constexpr (K == 8) {
        const float m = dpp_f<kHalfRowMirror>(v);  // lane ^ 7
        o[7] = m;
        o[6] = dpp_f<kQpXor1>(m);
        o[5] = dpp_f<kQpXor2>(m);
        o[4] = dpp_f<kQpXor3>(m);
    }
}

// o[p] = a[p] of lane (lane ^ p): with a[p] = A[c][c ^ p] (row c in xor
// order), o is row c of A^T in xor order, since A^T[c][c ^ p] = A[c ^ p][c]
// is entry p of lane c ^ p.
template <int K>
__device__ __forceinline__ void xor_each(const float (&a)[K], float (&o)[K]) {
    o[0] = a[0];
    o[1] = dpp_f<kQpXor1>(a[1]);
    o[2] = dpp_f<kQpXor2>(a[2]);
    o[3] = dpp_f<kQpXor3>(a[3]);
    if constexpr (K == 8) {
        o[7] = dpp_f<kHalfRowMirror>(a[7]);                   // lane ^ 7
        o[6] = dpp_f<kQpXor1>(dpp_f<kHalfRowMirror>(a[6]));  // lane ^ 7 ^ 1
        o[5] = dpp_f<kQpXor2>(dpp_f<kHalfRowMirror>(a[5]));  // lane ^ 7 ^ 2
        o[4] = dpp_f<kQpXor3>(dpp_f<kHalfRowMirror>(a[4]));  // lane ^ 7 ^ 3
    }
}

// 1 when every lane of the group has f = 1
template <int K>
__device__ __forceinline__ int group_all(int f) {
    f &= dpp_i<kQpXor1>(f);
    f &= dpp_i<kQpXor2>(f);
    if constexpr (K == 8) f &= dpp_i<kHalfRowMirror>(f);
    return f;
}

template <int K>
struct RowK {
    float a[K];  // a[p] = A[c][c ^ p]
    float b;     // b[c]
};

template <int K>
__device__ __forceinline__ RowK<K> row_id() {
    RowK<K> r;
#pragma unroll
    for (int p = 0; p < K; ++p) r.a[p] = p == 0 ? 1.0f : 0.0f;
    r.b = 0.0f;
    return r;
}

// o[p ^ q] += mul[p] * (v of lane (lane ^ p)) for p = 0..K-1: the terms
// that one value v of every lane of the group contributes.  With kBlkRowDppFma
// the lane exchange rides on the multiply-add itself (v_fmac_f32 with a DPP
// source operand; the compiler only folds DPP into v_mul/v_add, so this is
// written out), which halves the instructions of an exchange: K = 8 takes
// one mirror move and 7 DPP multiply-adds instead of 7 moves and 7
// multiply-adds.  A DPP source written by a VALU instruction needs two wait
// states before it is read, so each block starts with s_nop 1 (its source
// may have been written just before) and the mirror move is followed by one.
template <int K, int Q>
__device__ __forceinline__ void xor_terms(float v, const float (&mul)[K], float (&o)[K]) {
    if constexpr (kBlkRowDppFma) {
        o[Q] = fmaf(mul[0], v, o[Q]);
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %3, %4 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %3, %5 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, %3, %6 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf"
            : "+v"(o[Q ^ 1]), "+v"(o[Q ^ 2]), "+v"(o[Q ^ 3])
            : "v"(v), "v"(mul[1]), "v"(mul[2]), "v"(mul[3]));
        if constexpr (K == 8) {
            float m;
            asm("v_mov_b32_dpp %0, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
                "s_nop 1"
                : "=&v"(m)
                : "v"(v));
            o[Q ^ 7] = fmaf(mul[7], m, o[Q ^ 7]);
            asm("v_fmac_f32_dpp %0, %3, %4 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %1, %3, %5 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %2, %3, %6 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                : "+v"(o[Q ^ 4]), "+v"(o[Q ^ 5]), "+v"(o[Q ^ 6])
                : "v"(m), "v"(mul[4]), "v"(mul[5]), "v"(mul[6]));
        }
    } else {
        float x[K];
        xor_lanes<K>(v, x);
#pragma unroll
        for (int p = 0; p < K; ++p) o[p ^ Q] = fmaf(mul[p], x[p], o[p ^ Q]);
    }
}

// acc += sum_p mul[p] * (v of lane (lane ^ p)), the same exchange into one sum
template <int K>
__device__ __forceinline__ void xor_terms_sum(float v, const float (&mul)[K], float &acc) {
    if constexpr (kBlkRowDppFma) {
        acc = fmaf(mul[0], v, acc);
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %1, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %0, %1, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %0, %1, %4 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf"
            : "+v"(acc)
            : "v"(v), "v"(mul[1]), "v"(mul[2]), "v"(mul[3]));
        if constexpr (K == 8) {
            float m;
            asm("v_mov_b32_dpp %0, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
                "s_nop 1"
                : "=&v"(m)
                : "v"(v));
            acc = fmaf(mul[7], m, acc);
            asm("v_fmac_f32_dpp %0, %1, %2 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %0, %1, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
                "v_fmac_f32_dpp %0, %1, %4 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                : "+v"(acc)
                : "v"(m), "v"(mul[4]), "v"(mul[5]), "v"(mul[6]));
        }
    } else {
        float x[K];
        xor_lanes<K>(v, x);
#pragma unroll
        for (int p = 0; p < K; ++p) acc = fmaf(mul[p], x[p], acc);
    }
}

// o[p ^ Q] = mul[p] * (v of lane (lane ^ p)): the first exchange of a sum,
// which sets the terms instead of adding to zeroed ones.  Written with the
// DPP move builtins, which the compiler folds into the multiplies.
template <int K, int Q>
__device__ __forceinline__ void xor_terms_set(float v, const float (&mul)[K], float (&o)[K]) {
    o[Q] = mul[0] * v;
    o[Q ^ 1] = mul[1] * dpp_f<kQpXor1>(v);
    o[Q ^ 2] = mul[2] * dpp_f<kQpXor2>(v);
    o[Q ^ 3] = mul[3] * dpp_f<kQpXor3>(v);
    if constexpr (K == 8) {
        const float m = dpp_f<kHalfRowMirror>(v);  // lane ^ 7
        o[Q ^ 7] = mul[7] * m;
        o[Q ^ 6] = mul[6] * dpp_f<kQpXor1>(m);
        o[Q ^ 5] = mul[5] * dpp_f<kQpXor2>(m);
        o[Q ^ 4] = mul[4] * dpp_f<kQpXor3>(m);
    }
}

template <int K, int Q = 0>
__device__ __forceinline__ void then_cols(const RowK<K> &m1, const RowK<K> &m2, RowK<K> &r) {
    if constexpr (Q < K) {
        xor_terms<K, Q>(m1.a[Q], m2.a, r.a);
        then_cols<K, Q + 1>(m1, m2, r);
    }
}

// m2 after m1 (m1 applied first): (A2 A1, A2 b1 + b2)
template <int K>
__device__ __forceinline__ RowK<K> row_then(const RowK<K> &m1, const RowK<K> &m2) {
    RowK<K> r;
    xor_terms_set<K, 0>(m1.a[0], m2.a, r.a);
    then_cols<K, 1>(m1, m2, r);
    r.b = m2.b;
    xor_terms_sum<K>(m1.b, m2.a, r.b);
    return r;
}

// (A x + b)[c] for the state component x = x[c] of this lane
template <int K>
__device__ __forceinline__ float row_apply(const RowK<K> &m, float x) {
    float y = m.b;
    xor_terms_sum<K>(x, m.a, y);
    return y;
}

// Lane c of a 4-float piece v (v[i] = n[i]) -> v[i] = n[i ^ (c & 3)].
__device__ __forceinline__ void xor_order4(float (&v)[4], int c) {
    if (c & 1) {
        float t = v[0]; v[0] = v[1]; v[1] = t;
        t = v[2]; v[2] = v[3]; v[3] = t;
    }
    if (c & 2) {
        float t = v[0]; v[0] = v[2]; v[2] = t;
        t = v[1]; v[1] = v[3]; v[3] = t;
    }
}


struct Geo {
    int64_t B, L, H;          // H: heads (blocks) per batch row
    int64_t ncb, nq, ntiles;  // head blocks per batch row (64/K heads each), chunks, tiles
    int64_t nrow;             // rows per chunk: B * H * K
    WsSpan ws;
    uint64_t *agg, *inc;      // agg [nq][K + 1][nrow], inc [nq][nrow]
};

// Where a lane is: batch row b, head j (ok: it exists; uniform over the lane
// group), row c of the head's block, chunk q, first position pos0 of its
// sub-chunk (wave w of the workgroup).
struct Pos {
    int64_t b, j, q, pos0;
    int c, lane, w;
    bool ok;
};

template <class Op, int NW, int C>
__device__ __forceinline__ void scan_tile(const Op &op, const Geo &g, int64_t ticket, uint32_t tag) {
    constexpr int K = Op::K;
    constexpr int G = 64 / K;  // heads per wave
    constexpr int64_t T = (int64_t)NW * C;
    __shared__ float s_part[NW][K + 1][64];
    __shared__ float s_carry[64];

    Pos p;
    p.lane = threadIdx.x & 63;
    p.w = threadIdx.x >> 6;
    p.c = p.lane % K;
    const int64_t per_q = g.B * g.ncb;
    p.q = ticket / per_q;
    const int64_t rest = ticket - p.q * per_q;
    p.b = rest / g.ncb;
    p.j = (rest - p.b * g.ncb) * G + p.lane / K;
    p.ok = p.j < g.H;
    p.pos0 = p.q * T + (int64_t)p.w * C;
    const int lane = p.lane, w = p.w;

    typename Op::Elem e[C];
    const RowK<K> m = op.template phase1<C>(p, e);

    // sub-chunks of the chunk, earliest first
#pragma unroll
    for (int k = 0; k < K; ++k) s_part[w][k][lane] = m.a[k];
    s_part[w][K][lane] = m.b;
    __syncthreads();
    const bool holder = w == NW - 1;
    RowK<K> ex = row_id<K>();
    for (int k = 0; k < w; ++k) {
        RowK<K> o;
#pragma unroll
        for (int i = 0; i < K; ++i) o.a[i] = s_part[k][i][lane];
        o.b = s_part[k][K][lane];
        ex = k == 0 ? o : row_then<K>(ex, o);
    }

    if (holder) {
        const RowK<K> tot = w == 0 ? m : row_then<K>(ex, m);
        const int64_t slot = (p.b * g.H + p.j) * K + p.c;
        float xin = 0.0f;
        if (p.ok) {
            if (p.q == 0) {
                xin = op.init_state(p);
            } else {
                const int64_t d = p.q * (K + 1) * g.nrow + slot;
#pragma unroll
                for (int k = 0; k < K; ++k) st_coherent(g.agg + d + k * g.nrow, tagged(tot.a[k], tag));
                st_coherent(g.agg + d + K * g.nrow, tagged(tot.b, tag));
                // look-back, decided per lane group
                RowK<K> acc = row_id<K>();  // state entering predecessor pp+1 -> entering q
                int64_t pp = p.q - 1;
                uint32_t idle = 0;
                for (;;) {
                    const uint64_t wi = ld_coherent(g.inc + pp * g.nrow + slot);
                    uint64_t wa[K + 1];
                    const int64_t dp = pp * (K + 1) * g.nrow + slot;
#pragma unroll
                    for (int k = 0; k <= K; ++k) wa[k] = ld_coherent(g.agg + dp + k * g.nrow);
                    int ha = 1;
#pragma unroll
                    for (int k = 0; k <= K; ++k) ha &= has_tag(wa[k], tag) ? 1 : 0;
                    if (group_all<K>(has_tag(wi, tag) ? 1 : 0)) {
                        xin = row_apply<K>(acc, lo_f(wi));
                        break;
                    }
                    if (group_all<K>(ha)) {
                        RowK<K> mp;
#pragma unroll
                        for (int k = 0; k < K; ++k) mp.a[k] = lo_f(wa[k]);
                        mp.b = lo_f(wa[K]);
                        acc = row_then<K>(mp, acc);
                        --pp;  // chunk 0 publishes no aggregate, so pp stays >= 0
                        idle = 0;
                        continue;
                    }
                    if (++idle >= kMaxPolls) {
                        xin = __uint_as_float(0x7fc00000u);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            st_coherent(g.inc + p.q * g.nrow + slot, tagged(row_apply<K>(tot, xin), tag));
        }
        s_carry[lane] = xin;
    }
    __syncthreads();

    float x = s_carry[lane];
    if (w > 0) x = row_apply<K>(ex, x);
    op.template phase2<C, NW>(p, e, x);
}

// Persistent grid over the tiles in ticket order (as chunk_scan_kernel); a
// launch whose op is not active (a Newton iteration after convergence)
// returns at once.
template <class Op, int NW, int C, int MINW>
__global__ __launch_bounds__(NW * 64, MINW) void scan_kernel(Op op, Geo g) {
    __shared__ Ticket s_ticket;
    if (!op.active()) return;  // uniform over the grid
    const bool persistent = (int64_t)gridDim.x < g.ntiles;
    const uint32_t draws = (uint32_t)(persistent ? g.ntiles + gridDim.x : g.ntiles);
    for (;;) {
        if (threadIdx.x == 0) s_ticket = draw_ticket(g.ws.hdr, draws);
        __syncthreads();  // the tile's own barriers keep the next write after every read
        const Ticket t = s_ticket;
        if (t.index >= g.ntiles) {
            finish_launch(t, g.ws);
            return;
        }
        scan_tile<Op, NW, C>(op, g, t.index, t.tag);
        if (!persistent) {
            finish_launch(t, g.ws);
            return;
        }
    }
}

template <class Op, int NW, int C, int MINW>
hipError_t launch(const Op &op, const Geo &g, hipStream_t s) {
    static const int per_cu = blocks_per_cu(reinterpret_cast<const void *>(scan_kernel<Op, NW, C, MINW>), NW * 64);
    const int64_t slots = (int64_t)per_cu * device_cu_count();
    const int64_t grid = g.ntiles < slots ? g.ntiles : slots;
    hipLaunchKernelGGL((scan_kernel<Op, NW, C, MINW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, op, g);
    return hipGetLastError();
}

}  // namespace lg
}  // namespace prn
