// linscan.hip -- the exported linear-recurrence scans: the diagonal scan
// (channel lanes: its own persistent kernel that prefetches the next tile;
// time lanes: the generic chunked look-back scan of scan_core.hpp), the
// 2x2 and 4x4 block scans (scan_core.hpp), plus the small fill kernel that
// initialises info words, traces and per-iteration slots, and the device
// query shared by the launchers.
#include <atomic>

#include "launch.hpp"
#include "scan_core.hpp"

namespace prn {

// ---------------------------------------------------------------- fill
struct FillPack {
    FillRange r[kMaxFill];
    int n;
};

__global__ void fill_kernel(FillPack p) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (int k = 0; k < p.n; ++k) {
        const FillRange &r = p.r[k];
        for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < r.count; i += stride) {
            if (r.bytes == 8)
                static_cast<uint64_t *>(r.ptr)[i] = r.value;
            else
                static_cast<uint32_t *>(r.ptr)[i] = (uint32_t)r.value;
        }
    }
}

hipError_t fill(const FillRange *r, int n, hipStream_t s) {
    FillPack p;
    p.n = 0;
    uint64_t most = 0;
    for (int k = 0; k < n; ++k) {
        if (r[k].count == 0 || r[k].ptr == nullptr) continue;
        p.r[p.n++] = r[k];
        most = r[k].count > most ? r[k].count : most;
    }
    if (p.n == 0) return hipSuccess;
    uint64_t blocks = (most + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- diag scan
// h_t = a_t h_{t-1} + b_t per (batch, channel).
struct LinDiagOp {
    static constexpr int S = 1;
    const float *a, *b, *h0;
    float *h;
    int64_t L, H;

    struct Elem {
        float a, b;
    };
    __device__ bool active() const { return true; }
    __device__ float init_state(const TilePos &tp) const {
        return (h0 != nullptr && tp.ok) ? h0[tp.b * H + tp.j] : 0.0f;
    }
    template <int C>
    __device__ Aff1 phase1(const TilePos &tp, Elem (&e)[C]) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        if (tp.ok && tp.pos0 + C <= L) {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                e[i].a = ld_once(a + base + i * H);
                e[i].b = ld_once(b + base + i * H);
            }
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const bool v = tp.ok && tp.pos0 + i < L;
                e[i].a = v ? ld_once(a + base + i * H) : 1.0f;
                e[i].b = v ? ld_once(b + base + i * H) : 0.0f;
            }
        }
        Aff1 acc = {1.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < C; ++i) acc = {acc.a * e[i].a, fmaf(e[i].a, acc.b, e[i].b)};
        return acc;
    }
    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float x) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x = fmaf(e[i].a, x, e[i].b);
            if (tp.ok && tp.pos0 + i < L) h[base + i * H] = x;
        }
    }
};

// ---------------------------------------------------------------- 2x2 scan
// h_t = A_t h_{t-1} + b_t with A_t a 2x2 block per (batch, channel).  VEC:
// A 16-byte aligned, b, h and h0 8-byte aligned, so a block moves as one
// 16-byte access and a pair as one 8-byte access; otherwise every float is
// moved alone (any 4-byte aligned tensors).
template <bool VEC>
struct LinBlk2Op {
    static constexpr int S = 2;
    const float *A, *b, *h0;
    float *h;
    int64_t L, H;

    struct Elem {
        Aff2 m;
    };
    __device__ bool active() const { return true; }
    // the state before the first chunk of (batch row b, channel j)
    __device__ float2s init_at(int64_t b, int64_t j) const {
        if (h0 != nullptr) {
            const int64_t e = b * H + j;
            if (VEC) {
                const float2 v = reinterpret_cast<const float2 *>(h0)[e];
                return {v.x, v.y};
            }
            return {h0[2 * e], h0[2 * e + 1]};
        }
        return {0.0f, 0.0f};
    }
    __device__ float2s init_state(const TilePos &tp) const {
        return tp.ok ? init_at(tp.b, tp.j) : float2s{0.0f, 0.0f};
    }
    __device__ void load_elem(int64_t e, Aff2 &m) const {
        if (VEC) {
            const float4 a = ld_once(reinterpret_cast<const float4 *>(A) + e);
            const float2 v = ld_once(reinterpret_cast<const float2 *>(b) + e);
            m = {a.x, a.y, a.z, a.w, v.x, v.y};
        } else {
            m = {ld_once(A + 4 * e), ld_once(A + 4 * e + 1), ld_once(A + 4 * e + 2), ld_once(A + 4 * e + 3),
                 ld_once(b + 2 * e), ld_once(b + 2 * e + 1)};
        }
    }
    __device__ void store_state(int64_t e, float2s x) const {
        if (VEC) {
            reinterpret_cast<float2 *>(h)[e] = make_float2(x.x, x.y);
        } else {
            h[2 * e] = x.x;
            h[2 * e + 1] = x.y;
        }
    }
    template <int C>
    __device__ Aff2 phase1(const TilePos &tp, Elem (&e)[C]) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        if (tp.ok && tp.pos0 + C <= L) {  // every position inside: no test per position
#pragma unroll
            for (int i = 0; i < C; ++i) load_elem(base + i * H, e[i].m);
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                if (tp.ok && tp.pos0 + i < L)
                    load_elem(base + i * H, e[i].m);
                else
                    e[i].m = MonoidT<2>::id();
            }
        }
        Aff2 acc = e[0].m;
#pragma unroll
        for (int i = 1; i < C; ++i) acc = MonoidT<2>::then(acc, e[i].m);
        return acc;
    }
    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float2s x) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        if (tp.ok && tp.pos0 + C <= L) {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                x = MonoidT<2>::apply(e[i].m, x);
                store_state(base + i * H, x);
            }
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                x = MonoidT<2>::apply(e[i].m, x);
                if (tp.ok && tp.pos0 + i < L) store_state(base + i * H, x);
            }
        }
    }
};

// ---------------------------------------------------------------- scans, prefetching
// The diagonal and 2x2 scans with channel lanes, as a persistent kernel that
// keeps the next tile's inputs in flight while the current tile finishes.  A
// tile is the scan_core.hpp channel-lane tile (NWC groups of 64 channels x
// NW/NWC sub-chunks of C positions).  Each workgroup draws its next ticket
// while it composes the current tile; after the first barrier every wave
// issues the loads of the next tile into a second register set, so they
// overlap the look-back, the second barrier, the carry-in and the stores of
// the current one.  The holder waves issue theirs after their look-back:
// loads complete in issue order, so look-back loads queued behind them would
// wait for them.  The two register sets alternate by unrolling the tile loop
// twice.  Every wait is still on a smaller ticket (a workgroup finishes its
// tiles in ticket order), and each workgroup draws exactly one ticket past the
// last tile.
struct PfTilePos {
    int64_t q, b, j, pos0, base;
    bool ok;
};

template <int NW, int C, int NWC>
__device__ __forceinline__ PfTilePos pf_tile_pos(const ScanGeo &g, int64_t ticket) {
    constexpr int NWT = NW / NWC;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cw = w % NWC, tw = w / NWC;
    PfTilePos p;
    const int64_t per_q = g.B * g.ncb;
    p.q = ticket / per_q;
    const int64_t rest = ticket - p.q * per_q;
    p.b = rest / g.ncb;
    const int64_t cb = rest - p.b * g.ncb;
    p.j = (cb * NWC + cw) * 64 + lane;
    p.ok = p.j < g.H;
    p.pos0 = p.q * ((int64_t)NWT * C) + (int64_t)tw * C;
    p.base = idx3(p.b, p.pos0, p.ok ? p.j : 0, g.L, g.H);
    return p;
}

// The op-specific pieces: a tile's maps (the identity outside the sequence),
// the state before the first chunk, and the stores.
template <int C>
__device__ __forceinline__ void pf_load(const LinDiagOp &op, const PfTilePos &p, Aff1 (&m)[C]) {
    if (p.ok && p.pos0 + C <= op.L) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            m[i].a = ld_once(op.a + p.base + i * op.H);
            m[i].b = ld_once(op.b + p.base + i * op.H);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const bool v = p.ok && p.pos0 + i < op.L;
            m[i].a = v ? ld_once(op.a + p.base + i * op.H) : 1.0f;
            m[i].b = v ? ld_once(op.b + p.base + i * op.H) : 0.0f;
        }
    }
}
__device__ __forceinline__ float pf_init(const LinDiagOp &op, const PfTilePos &p) {
    return op.h0 != nullptr ? op.h0[p.b * op.H + p.j] : 0.0f;
}
__device__ __forceinline__ void pf_store(const LinDiagOp &op, int64_t e, float x) { op.h[e] = x; }

template <int C, bool VEC>
__device__ __forceinline__ void pf_load(const LinBlk2Op<VEC> &op, const PfTilePos &p, Aff2 (&m)[C]) {
    if (p.ok && p.pos0 + C <= op.L) {
#pragma unroll
        for (int i = 0; i < C; ++i) op.load_elem(p.base + i * op.H, m[i]);
    } else {
        // every load issued, none behind a branch (a position outside reads
        // element 0 and takes the identity by selects)
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const bool v = p.ok && p.pos0 + i < op.L;
            op.load_elem(v ? p.base + i * op.H : 0, m[i]);
            const Aff2 id = MonoidT<2>::id();
            m[i] = {v ? m[i].a00 : id.a00, v ? m[i].a01 : id.a01, v ? m[i].a10 : id.a10,
                    v ? m[i].a11 : id.a11, v ? m[i].b0 : id.b0,   v ? m[i].b1 : id.b1};
        }
    }
}
template <bool VEC>
__device__ __forceinline__ float2s pf_init(const LinBlk2Op<VEC> &op, const PfTilePos &p) {
    return op.init_at(p.b, p.j);
}
template <bool VEC>
__device__ __forceinline__ void pf_store(const LinBlk2Op<VEC> &op, int64_t e, float2s x) {
    op.store_state(e, x);
}

// One tile (inputs already in m); prefetches the next ticket's tile into nm.
// Returns whether there is a next tile.
template <class Op, int NW, int C, int NWC>
__device__ __forceinline__ bool pf_tile(const Op &op, const ScanGeo &g, uint32_t draws, const PfTilePos &p,
                                        uint32_t tag, typename MonoidT<Op::S>::Map (&m)[C], Ticket *s_next,
                                        typename MonoidT<Op::S>::Map *s_part,
                                        typename MonoidT<Op::S>::State *s_carry, PfTilePos &pn,
                                        typename MonoidT<Op::S>::Map (&nm)[C], Ticket &tn) {
    using M = MonoidT<Op::S>;
    using D = Desc<Op::S>;
    using Map = typename M::Map;
    using State = typename M::State;
    constexpr int NWT = NW / NWC;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cw = w % NWC, tw = w / NWC;
    const bool holder = tw == NWT - 1;
    const int cslot = cw * 64 + lane;

    Map acc = M::id();
#pragma unroll
    for (int i = 0; i < C; ++i) acc = M::then(acc, m[i]);
    if (tid == 0) *s_next = draw_ticket(g.ws.hdr, draws);
    s_part[w * 64 + lane] = acc;
    lds_barrier();
    tn = *s_next;
    const bool more = tn.index < g.ntiles;
    if (more) pn = pf_tile_pos<NW, C, NWC>(g, tn.index);
    if (more && !holder) pf_load<C>(op, pn, nm);

    Map ex = M::id();
    for (int k = 0; k < tw; ++k) ex = M::then(ex, s_part[(k * NWC + cw) * 64 + lane]);
    if (holder) {
        const Map tot = M::then(ex, acc);
        const int64_t stride = g.B * g.H, slot = p.b * g.H + p.j;
        const int64_t dsc = p.q * stride + slot;
        State xin = M::zero();
        if (p.ok) {
            if (p.q == 0) {
                xin = pf_init(op, p);
            } else {
                D::put_agg(g.agg + dsc * D::kAggWords, tot, tag);
                xin = lane_lookback<Op::S>(g, tag, p.q, stride, slot);
            }
            D::put_inc(g.inc + dsc * D::kIncWords, M::apply(tot, xin), tag);
        }
        s_carry[cslot] = xin;
        if (more) pf_load<C>(op, pn, nm);
    }
    lds_barrier();

    State x = M::apply(ex, s_carry[cslot]);
    if (p.ok && p.pos0 + C <= op.L) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x = M::apply(m[i], x);
            pf_store(op, p.base + i * op.H, x);
        }
    } else {
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x = M::apply(m[i], x);
            if (p.ok && p.pos0 + i < op.L) pf_store(op, p.base + i * op.H, x);
        }
    }
    return more;
}

template <class Op, int NW, int C, int NWC>
__global__ __launch_bounds__(NW * 64) void scan_pf_kernel(Op op, ScanGeo g) {
    static_assert(NW % NWC == 0, "channel groups tile the waves");
    using M = MonoidT<Op::S>;
    __shared__ typename M::Map s_part[NW * 64];
    __shared__ typename M::State s_carry[64 * NWC];
    __shared__ Ticket s_tk[2];
    const uint32_t draws = (uint32_t)(g.ntiles + gridDim.x);  // one draw past the end per workgroup
    if (threadIdx.x == 0) s_tk[0] = draw_ticket(g.ws.hdr, draws);
    __syncthreads();
    Ticket tx = s_tk[0], ty;
    if (tx.index >= g.ntiles) {
        finish_launch(tx, g.ws);
        return;
    }
    PfTilePos px = pf_tile_pos<NW, C, NWC>(g, tx.index), py;
    typename M::Map xm[C], ym[C];
    pf_load<C>(op, px, xm);
    for (;;) {
        if (!pf_tile<Op, NW, C, NWC>(op, g, draws, px, tx.tag, xm, &s_tk[1], s_part, s_carry, py, ym, ty)) break;
        if (!pf_tile<Op, NW, C, NWC>(op, g, draws, py, ty.tag, ym, &s_tk[0], s_part, s_carry, px, xm, tx)) break;
    }
    finish_launch(tx, g.ws);  // every draw of a launch carries the same epoch
}

template <class Op, int NW, int C, int NWC>
static hipError_t launch_scan_pf(const Op &op, const ScanGeo &g, hipStream_t s) {
    static const int per_cu = blocks_per_cu(reinterpret_cast<const void *>(scan_pf_kernel<Op, NW, C, NWC>), NW * 64);
    const int64_t slots = (int64_t)per_cu * device_cu_count();
    const int64_t grid = g.ntiles < slots ? g.ntiles : slots;
    hipLaunchKernelGGL((scan_pf_kernel<Op, NW, C, NWC>), dim3((unsigned)grid), dim3(NW * 64), 0, s, op, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------- k x k scan
// h_t = A_t h_{t-1} + b_t with A_t a dense k x k block per (batch, channel):
// the 2x2 case widened to the small dense blocks that dense Jacobians per
// head give (ParaRNN page, Fig. 2 caption: block bi-diagonal systems; DEER
// summary page, limitations: dense Jacobians).  VEC: every tensor 16-byte
// aligned, so block rows and states move as whole 16-byte pieces; otherwise
// every float is moved alone.  Instantiated for k = 4: one thread holds
// k*k + k floats per position.
template <int K, bool VEC>
struct LinBlkOp {
    static_assert(K % 4 == 0, "blocks move as float4s");
    static constexpr int S = K;
    using M = MonoidT<K>;
    const float *A, *b, *h0;
    float *h;
    int64_t L, H;

    struct Elem {
        AffK<K> m;
    };
    __device__ bool active() const { return true; }
    __device__ static void load_vec(const float *p, float *v) {
        if (VEC) {
#pragma unroll
            for (int q = 0; q < K / 4; ++q) {
                const float4 x = reinterpret_cast<const float4 *>(p)[q];
                v[4 * q] = x.x;
                v[4 * q + 1] = x.y;
                v[4 * q + 2] = x.z;
                v[4 * q + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < K; ++q) v[q] = p[q];
        }
    }
    __device__ VecK<K> init_state(const TilePos &tp) const {
        VecK<K> x = M::zero();
        if (h0 != nullptr && tp.ok) load_vec(h0 + (tp.b * H + tp.j) * K, x.v);
        return x;
    }
    // map of element e = (b, t, j): its block and offsets.  A lane's block is
    // 64 consecutive bytes, half a line, read as four 16-byte pieces: ordinary
    // loads there (the streamed hint took 322 us against 264 us at B=16,
    // L=2048, H=256); the offsets are streamed.
    __device__ void load_elem(int64_t e, AffK<K> &m) const {
        if (VEC) {
            const float4 *a4 = reinterpret_cast<const float4 *>(A) + e * (K * K / 4);
#pragma unroll
            for (int q = 0; q < K * K / 4; ++q) {
                const float4 x = a4[q];
                m.a[4 * q] = x.x;
                m.a[4 * q + 1] = x.y;
                m.a[4 * q + 2] = x.z;
                m.a[4 * q + 3] = x.w;
            }
            const float4 *b4 = reinterpret_cast<const float4 *>(b) + e * (K / 4);
#pragma unroll
            for (int q = 0; q < K / 4; ++q) {
                const float4 x = ld_once(b4 + q);
                m.b[4 * q] = x.x;
                m.b[4 * q + 1] = x.y;
                m.b[4 * q + 2] = x.z;
                m.b[4 * q + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < K * K; ++q) m.a[q] = A[e * (K * K) + q];
#pragma unroll
            for (int q = 0; q < K; ++q) m.b[q] = ld_once(b + e * K + q);
        }
    }
    template <int C>
    __device__ AffK<K> phase1(const TilePos &tp, Elem (&e)[C]) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        if (tp.ok && tp.pos0 + C <= L) {  // every position inside: no test per position
#pragma unroll
            for (int i = 0; i < C; ++i) load_elem(base + i * H, e[i].m);
        } else {
#pragma unroll
            for (int i = 0; i < C; ++i) {
                if (tp.ok && tp.pos0 + i < L)
                    load_elem(base + i * H, e[i].m);
                else
                    e[i].m = M::id();
            }
        }
        AffK<K> acc = e[0].m;
#pragma unroll
        for (int i = 1; i < C; ++i) acc = M::then(acc, e[i].m);
        return acc;
    }
    __device__ void store_state(int64_t e, const VecK<K> &x) const {
        if (VEC) {
            float4 *h4 = reinterpret_cast<float4 *>(h) + e * (K / 4);
#pragma unroll
            for (int q = 0; q < K / 4; ++q)
                h4[q] = make_float4(x.v[4 * q], x.v[4 * q + 1], x.v[4 * q + 2], x.v[4 * q + 3]);
        } else {
#pragma unroll
            for (int q = 0; q < K; ++q) h[e * K + q] = x.v[q];
        }
    }
    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], VecK<K> x) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x = M::apply(e[i].m, x);
            if (tp.ok && tp.pos0 + i < L) store_state(base + i * H, x);
        }
    }
};

int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int blocks_per_cu(const void *kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0) n = 1;
    return n;
}

template <class Op, int S, int NWC, int CC, int NWT, int CT, int NCW>
static hipError_t run_scan(const TileCfg &cfg, const Op &op, int64_t B, int64_t L, int64_t H,
                           const Ws &ws, hipStream_t s) {
    const ScanWs w = scan_ws(cfg, S, B, L, H);
    ScanGeo g;
    g.B = B;
    g.L = L;
    g.H = H;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.ws = ws_span(ws);
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    return w.sh.channel_lanes ? launch_chunk_scan<Op, NWC, CC, true, NCW>(op, g, s)
                              : launch_chunk_scan<Op, NWT, CT, false>(op, g, s);
}

// The prefetching form (channel lanes only) on the same workspace layout.
template <class Op, int NW, int C, int NWC>
static hipError_t run_scan_pf(const TileCfg &cfg, const Op &op, int64_t B, int64_t L, int64_t H, const Ws &ws,
                              hipStream_t s) {
    const ScanWs w = scan_ws(cfg, Op::S, B, L, H);
    ScanGeo g;
    g.B = B;
    g.L = L;
    g.H = H;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.ws = ws_span(ws);
    g.agg = reinterpret_cast<uint64_t *>(ws.p + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws.p + w.inc);
    return launch_scan_pf<Op, NW, C, NWC>(op, g, s);
}


hipError_t linscan_diag(int64_t B, int64_t L, int64_t H, const float *a, const float *b,
                        const float *h0, float *h, const Ws &ws, hipStream_t s) {
    LinDiagOp op{a, b, h0, h, L, H};
    constexpr TileCfg c = kCfgLinDiag;
    if (kDiagPrefetch && H >= kChannelLanesMinH) return run_scan_pf<LinDiagOp, c.nw_cl, c.c_cl, c.ncw_cl>(c, op, B, L, H, ws, s);
    return run_scan<LinDiagOp, 1, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
}

hipError_t linscan_blk2(int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                        const float *h0, float *h, const Ws &ws, hipStream_t s) {
    constexpr TileCfg c = kCfgLinBlk2;
    const bool vec = aligned16(A) && aligned_to(b, 8) && aligned_to(h, 8) && (h0 == nullptr || aligned_to(h0, 8));
    const bool pf = kBlk2Prefetch && H >= kChannelLanesMinH;
    if (vec) {
        LinBlk2Op<true> op{A, b, h0, h, L, H};
        if (pf) return run_scan_pf<LinBlk2Op<true>, c.nw_cl, c.c_cl, c.ncw_cl>(c, op, B, L, H, ws, s);
        return run_scan<LinBlk2Op<true>, 2, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
    }
    LinBlk2Op<false> op{A, b, h0, h, L, H};
    if (pf) return run_scan_pf<LinBlk2Op<false>, c.nw_cl, c.c_cl, c.ncw_cl>(c, op, B, L, H, ws, s);
    return run_scan<LinBlk2Op<false>, 2, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
}

hipError_t linscan_blk(int k, int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                       const float *h0, float *h, const Ws &ws, hipStream_t s) {
    if (k == 4) {
        constexpr TileCfg c = kCfgLinBlk4;
        const bool vec = aligned16(A) && aligned16(b) && aligned16(h) && (h0 == nullptr || aligned16(h0));
        if (vec) {
            LinBlkOp<4, true> op{A, b, h0, h, L, H};
            return run_scan<LinBlkOp<4, true>, 4, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
        }
        LinBlkOp<4, false> op{A, b, h0, h, L, H};
        return run_scan<LinBlkOp<4, false>, 4, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace prn
