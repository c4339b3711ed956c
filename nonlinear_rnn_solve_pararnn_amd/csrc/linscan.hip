// linscan.hip -- the exported linear-recurrence scans (diagonal and 2x2
// block) on the chunked look-back scan of scan_core.hpp, plus the small fill
// kernel that initialises info words, traces and per-iteration slots, and
// the device query shared by the launchers.
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
// h_t = A_t h_{t-1} + b_t with A_t a 2x2 block per (batch, channel).
struct LinBlk2Op {
    static constexpr int S = 2;
    const float *A, *b, *h0;
    float *h;
    int64_t L, H;

    struct Elem {
        Aff2 m;
    };
    __device__ bool active() const { return true; }
    __device__ float2s init_state(const TilePos &tp) const {
        if (h0 != nullptr && tp.ok) {
            const float2 v = reinterpret_cast<const float2 *>(h0)[tp.b * H + tp.j];
            return {v.x, v.y};
        }
        return {0.0f, 0.0f};
    }
    template <int C>
    __device__ Aff2 phase1(const TilePos &tp, Elem (&e)[C]) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        const float4 *A4 = reinterpret_cast<const float4 *>(A);
        const float2 *b2 = reinterpret_cast<const float2 *>(b);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            if (tp.ok && tp.pos0 + i < L) {
                const float4 m = ld_once(A4 + base + i * H);
                const float2 v = ld_once(b2 + base + i * H);
                e[i].m = {m.x, m.y, m.z, m.w, v.x, v.y};
            } else {
                e[i].m = MonoidT<2>::id();
            }
        }
        Aff2 acc = MonoidT<2>::id();
#pragma unroll
        for (int i = 0; i < C; ++i) acc = MonoidT<2>::then(acc, e[i].m);
        return acc;
    }
    template <int C, int NW, bool CL>
    __device__ void phase2(const TilePos &tp, Elem (&e)[C], float2s x) const {
        const int64_t base = idx3(tp.b, tp.pos0, tp.j, L, H);
        float2 *h2 = reinterpret_cast<float2 *>(h);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            x = MonoidT<2>::apply(e[i].m, x);
            if (tp.ok && tp.pos0 + i < L) h2[base + i * H] = make_float2(x.x, x.y);
        }
    }
};

int device_cu_count() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <class Op, int S, int NWC, int CC, int NWT, int CT, int NCW>
static hipError_t run_scan(const TileCfg &cfg, const Op &op, int64_t B, int64_t L, int64_t H,
                           char *ws, hipStream_t s) {
    const ScanWs w = scan_ws(cfg, S, B, L, H);
    ScanGeo g;
    g.B = B;
    g.L = L;
    g.H = H;
    g.ncb = w.sh.ncb;
    g.nq = w.sh.nq;
    g.ntiles = w.sh.ntiles;
    g.hdr = reinterpret_cast<uint64_t *>(ws + w.hdr);
    g.agg = reinterpret_cast<uint64_t *>(ws + w.agg);
    g.inc = reinterpret_cast<uint64_t *>(ws + w.inc);
    return w.sh.channel_lanes ? launch_chunk_scan<Op, NWC, CC, true, NCW>(op, g, s)
                              : launch_chunk_scan<Op, NWT, CT, false>(op, g, s);
}


hipError_t linscan_diag(int64_t B, int64_t L, int64_t H, const float *a, const float *b,
                        const float *h0, float *h, char *ws, hipStream_t s) {
    LinDiagOp op{a, b, h0, h, L, H};
    constexpr TileCfg c = kCfgLinDiag;
    return run_scan<LinDiagOp, 1, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
}

hipError_t linscan_blk2(int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                        const float *h0, float *h, char *ws, hipStream_t s) {
    LinBlk2Op op{A, b, h0, h, L, H};
    constexpr TileCfg c = kCfgLinBlk2;
    return run_scan<LinBlk2Op, 2, c.nw_cl, c.c_cl, c.nw_tl, c.c_tl, c.ncw_cl>(c, op, B, L, H, ws, s);
}

}  // namespace prn
