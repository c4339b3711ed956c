// plan.hpp -- host-side geometry of every launch and the layout of the
// caller's workspace.  The workspace query and the dispatch both use these
// functions, so the size reported is exactly the size used.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace prn {

// Tile shapes (waves per workgroup, positions per thread) for the two lane
// mappings of scan_core.hpp.  The kernels are instantiated with exactly these.
struct TileCfg {
    int nw_cl, c_cl;  // channel lanes (H >= 32)
    int nw_tl, c_tl;  // time lanes (H < 32)
    int ncw_cl = 1;   // channel lanes: groups of 64 channels per workgroup
};
constexpr TileCfg kCfgLinDiag{16, 16, 4, 16, 2};
// The diagonal scan with channel lanes prefetches the next tile (linscan.hip).
constexpr bool kDiagPrefetch = true;
constexpr TileCfg kCfgLinBlk2{16, 8, 4, 8, 1};
// 4x4 blocks (the maps hold 20 floats per position)
constexpr TileCfg kCfgLinBlk4{8, 4, 4, 2, 1};
constexpr TileCfg kCfgGruStep{4, 16, 8, 16};
constexpr TileCfg kCfgLstmStep{8, 16, 4, 8};
constexpr TileCfg kCfgGruAdj{4, 8, 16, 8};
constexpr TileCfg kCfgLstmAdj{8, 16, 4, 4};
constexpr TileCfg kCfgGruChain{4, 16, 8, 24};
constexpr TileCfg kCfgLstmChain{8, 8, 8, 8};
// Channel-lane tiles of the chained kernel's form in which workgroups own
// whole chains (its time-lane fields are unused).
constexpr TileCfg kCfgGruLocal{16, 8, 8, 16};
constexpr TileCfg kCfgLstmLocal{8, 8, 8, 8};
// Waves per SIMD the chained kernels are compiled for (bounds their registers).
constexpr int kChainMinWaves = 1;
// Largest Newton cap the chained kernels take (their workspace holds the
// records of every iteration).
constexpr int32_t kChainMaxCap = 64;
// Only the exported scans use channel groups: the Newton and adjoint ops
// reduce over all waves of a workgroup as if they were one channel group.
static_assert(kCfgGruStep.ncw_cl == 1 && kCfgLstmStep.ncw_cl == 1 && kCfgGruAdj.ncw_cl == 1 &&
                  kCfgLstmAdj.ncw_cl == 1 && kCfgGruChain.ncw_cl == 1 && kCfgLstmChain.ncw_cl == 1 &&
                  kCfgGruLocal.ncw_cl == 1 && kCfgLstmLocal.ncw_cl == 1,
              "channel groups are for the exported scans only");
constexpr int64_t kChannelLanesMinH = 32;
// Look-back descriptors polled at once by one channel lane (diagonal, 2x2;
// batches of 2 to 8 measured slower with the current tiles).
constexpr int kLbBatchDiag = 1;
constexpr int kLbBatchBlk2 = 1;
// Scan launches use a grid of as many workgroups as fit on the device at
// once, each drawing tiles until none is left (instead of one per tile).
constexpr bool kScanPersistent = true;

struct ScanShape {
    bool channel_lanes;
    int nw, c;
    int64_t T;       // positions per chunk
    int64_t ncb;     // channel blocks per batch row
    int64_t nq;      // chunks along the sequence
    int64_t ntiles;  // workgroups per launch
    int64_t ndesc;   // look-back descriptors (nq * B * H)
};

inline ScanShape scan_shape(const TileCfg &cfg, int64_t B, int64_t L, int64_t H) {
    ScanShape s;
    s.channel_lanes = H >= kChannelLanesMinH;
    s.nw = s.channel_lanes ? cfg.nw_cl : cfg.nw_tl;
    s.c = s.channel_lanes ? cfg.c_cl : cfg.c_tl;
    const int64_t width = s.channel_lanes ? (int64_t)64 * cfg.ncw_cl : 1;  // channels per tile
    s.T = s.channel_lanes ? (int64_t)(s.nw / cfg.ncw_cl) * s.c : (int64_t)s.nw * 64 * s.c;
    s.ncb = s.channel_lanes ? (H + width - 1) / width : H;
    s.nq = (L + s.T - 1) / s.T;
    s.ntiles = s.nq * B * s.ncb;
    s.ndesc = s.nq * B * H;
    return s;
}

// Bump allocator over the workspace (256-byte aligned sections).
struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    }
};

// Every workspace starts with the 8-byte ticket header (common.hpp), at the
// same offset for every entry point, so one zero-filled buffer can serve any
// sequence of calls.

// 64-bit words of one look-back descriptor of a recurrence with S state
// components: the aggregate map (S x S matrix and S offsets) and the
// inclusive state.
constexpr int desc_agg_words(int S) { return S * S + S; }
constexpr int desc_inc_words(int S) { return S; }

// Workspace of one scan launch: header and one descriptor set.
struct ScanWs {
    ScanShape sh;
    size_t hdr, agg, inc, partial, total;
};

inline ScanWs scan_ws(const TileCfg &cfg, int S, int64_t B, int64_t L, int64_t H,
                      int64_t partial_floats_per_tile = 0) {
    ScanWs w;
    w.sh = scan_shape(cfg, B, L, H);
    Carve c;
    w.hdr = c.take(8);
    w.agg = c.take((size_t)w.sh.ndesc * desc_agg_words(S) * 8);
    w.inc = c.take((size_t)w.sh.ndesc * desc_inc_words(S) * 8);
    w.partial = c.take((size_t)w.sh.ntiles * partial_floats_per_tile * 4);
    w.total = c.off;
    return w;
}

// Workspace of the per-iteration Newton path: header, a max|delta| slot per
// iteration, one descriptor set (launch tags tell the launches apart) and
// two sets of chunk-boundary states (state components `S`), used
// alternately by consecutive iterations.
struct NewtonWs {
    ScanShape sh;
    size_t hdr, maxd, agg, inc, bnd[2], total;
};

inline NewtonWs newton_ws(const TileCfg &cfg, int S, int64_t B, int64_t L, int64_t H,
                          int32_t cap) {
    NewtonWs w;
    w.sh = scan_shape(cfg, B, L, H);
    Carve c;
    w.hdr = c.take(8);
    w.maxd = c.take((size_t)cap * 4);
    w.agg = c.take((size_t)w.sh.ndesc * desc_agg_words(S) * 8);
    w.inc = c.take((size_t)w.sh.ndesc * desc_inc_words(S) * 8);
    for (int k = 0; k < 2; ++k) w.bnd[k] = c.take((size_t)w.sh.ndesc * S * 4);
    w.total = c.off;
    return w;
}

// Workspace of the chained Newton kernel: header, the records of every
// iteration (aggregate and inclusive delta of each chunk and channel), a stop
// word per tile and per-iteration converged flags per tile.
struct ChainWs {
    ScanShape sh;
    size_t hdr, agg, inc, stop, fagg, finc, total;
};

inline ChainWs chain_ws(const TileCfg &cfg, int S, int64_t B, int64_t L, int64_t H, int32_t cap) {
    ChainWs w;
    w.sh = scan_shape(cfg, B, L, H);
    Carve c;
    w.hdr = c.take(8);
    w.agg = c.take((size_t)cap * w.sh.ndesc * desc_agg_words(S) * 8);
    w.inc = c.take((size_t)cap * w.sh.ndesc * desc_inc_words(S) * 8);
    w.stop = c.take((size_t)w.sh.ntiles * 8);
    w.fagg = c.take((size_t)cap * w.sh.ntiles * 8);
    w.finc = c.take((size_t)cap * w.sh.ntiles * 8);
    w.total = c.off;
    return w;
}

// Fused on-chip GRU Newton: one workgroup owns all L positions of
// kFusedChannels channels of one batch row; each lane is one (channel,
// sub-chunk), 32 sub-chunks of C positions (so 32 * kFusedChannels / 64
// waves).  Usable while L <= 32 * 16.  kFusedXcdOrder gives each XCD a
// contiguous run of tiles.
constexpr int kFusedChannels = 16;
constexpr bool kFusedXcdOrder = true;
constexpr int kFusedSubchunks = 32;
constexpr int kFusedMaxC = 16;
constexpr int64_t kFusedMaxL = (int64_t)kFusedSubchunks * kFusedMaxC;

inline int fused_c_for(int64_t L) {
    for (int c = 1; c <= kFusedMaxC; c *= 2)
        if (L <= (int64_t)kFusedSubchunks * c) return c;
    return 0;
}

}  // namespace prn
