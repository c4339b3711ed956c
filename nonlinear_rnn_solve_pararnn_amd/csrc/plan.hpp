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
    int cw_cl = 64;   // channel lanes: channels per wave row (32: a wave holds two sub-chunks)
};
constexpr TileCfg kCfgLinDiag{16, 16, 4, 16, 2};
// The diagonal scan with channel lanes prefetches the next tile (linscan.hip).
constexpr bool kDiagPrefetch = true;
constexpr TileCfg kCfgLinBlk2{8, 12, 4, 8, 1};
// The 2x2 scan with channel lanes prefetches the next tile too.
constexpr bool kBlk2Prefetch = true;
// 4x4 blocks (the maps hold 20 floats per position)
constexpr TileCfg kCfgLinBlk4{8, 4, 4, 2, 1};
constexpr TileCfg kCfgGruStep{4, 16, 8, 16};
constexpr TileCfg kCfgLstmStep{8, 16, 4, 8};
constexpr TileCfg kCfgGruAdj{4, 8, 16, 8};
constexpr TileCfg kCfgLstmAdj{8, 16, 4, 4};
constexpr TileCfg kCfgGruChain{4, 16, 8, 28};
constexpr TileCfg kCfgLstmChain{8, 8, 8, 8};
// Channel-lane tiles of the chained kernel's form in which workgroups own
// whole chains (its time-lane fields are unused).  The LSTM's chains are 32
// channels wide, so that two 4-wave workgroups share a CU and each one's
// serial phases overlap the other's cells.
constexpr TileCfg kCfgGruLocal{16, 8, 8, 16};
constexpr TileCfg kCfgLstmLocal{4, 8, 8, 8, 1, 32};
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
static_assert(kCfgGruStep.cw_cl == 64 && kCfgLstmStep.cw_cl == 64 && kCfgGruAdj.cw_cl == 64 &&
                  kCfgLstmAdj.cw_cl == 64 && kCfgGruChain.cw_cl == 64 && kCfgLstmChain.cw_cl == 64 &&
                  kCfgLinDiag.cw_cl == 64 && kCfgLinBlk2.cw_cl == 64 && kCfgLinBlk4.cw_cl == 64,
              "half-wave channel rows are for the whole-chain form only");
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
    const int64_t width = s.channel_lanes ? (int64_t)cfg.cw_cl * cfg.ncw_cl : 1;  // channels per tile
    s.T = s.channel_lanes ? (int64_t)(s.nw / cfg.ncw_cl) * (64 / cfg.cw_cl) * s.c : (int64_t)s.nw * 64 * s.c;
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

// Every workspace starts with the 16-byte ticket header (tags.hpp), at the
// same offset for every entry point, so one zero-filled buffer can serve any
// sequence of calls.

// 64-bit words of one look-back descriptor of a recurrence with S state
// components: the aggregate map (S x S matrix and S offsets) and the
// inclusive state.
constexpr int desc_agg_words(int S) { return S * S + S; }
constexpr int desc_inc_words(int S) { return S; }

// Workspace of one scan launch: header, the per-tile partial sums of the
// adjoint's dL/du (read by a later launch of the same call, so the clear at
// the end of a tag period keeps them: [partial, keep_end)) and one
// descriptor set.
struct ScanWs {
    ScanShape sh;
    size_t hdr, partial, keep_end, agg, inc, total;
};

inline ScanWs scan_ws(const TileCfg &cfg, int S, int64_t B, int64_t L, int64_t H,
                      int64_t partial_floats_per_tile = 0) {
    ScanWs w;
    w.sh = scan_shape(cfg, B, L, H);
    Carve c;
    w.hdr = c.take(16);
    w.partial = c.take((size_t)w.sh.ntiles * partial_floats_per_tile * 4);
    w.keep_end = c.off;
    w.agg = c.take((size_t)w.sh.ndesc * desc_agg_words(S) * 8);
    w.inc = c.take((size_t)w.sh.ndesc * desc_inc_words(S) * 8);
    w.total = c.off;
    return w;
}

// Workspace of the per-iteration Newton path: header, a max|delta| slot per
// iteration and two sets of chunk-boundary states (state components `S`),
// used alternately by consecutive iterations (state that later launches of
// the call read: [maxd, keep_end)), then one descriptor set (launch tags
// tell the launches apart).
struct NewtonWs {
    ScanShape sh;
    size_t hdr, maxd, bnd[2], keep_end, agg, inc, total;
};

inline NewtonWs newton_ws(const TileCfg &cfg, int S, int64_t B, int64_t L, int64_t H,
                          int32_t cap) {
    NewtonWs w;
    w.sh = scan_shape(cfg, B, L, H);
    Carve c;
    w.hdr = c.take(16);
    w.maxd = c.take((size_t)cap * 4);
    for (int k = 0; k < 2; ++k) w.bnd[k] = c.take((size_t)w.sh.ndesc * S * 4);
    w.keep_end = c.off;
    w.agg = c.take((size_t)w.sh.ndesc * desc_agg_words(S) * 8);
    w.inc = c.take((size_t)w.sh.ndesc * desc_inc_words(S) * 8);
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
    w.hdr = c.take(16);
    w.agg = c.take((size_t)cap * w.sh.ndesc * desc_agg_words(S) * 8);
    w.inc = c.take((size_t)cap * w.sh.ndesc * desc_inc_words(S) * 8);
    w.stop = c.take((size_t)w.sh.ntiles * 8);
    w.fagg = c.take((size_t)cap * w.sh.ntiles * 8);
    w.finc = c.take((size_t)cap * w.sh.ntiles * 8);
    w.total = c.off;
    return w;
}

// k x k blocks (k = 4, 8) with each block's rows on a group of k lanes
// (blkrow.hip): a wave holds 64/k heads, a workgroup nw waves that are
// consecutive sub-chunks of c positions of the same heads.
struct BlkRowCfg {
    int nw, c;
    int minw;  // waves per SIMD the kernel's registers must allow
};
// Measured at B=16, L=2048 (8x8: H=64 heads, 4x4: H=256) with branch-free
// loads: 8x8 with 4 waves x 7 positions bounded to 168 registers (three
// workgroups per CU, no spills in the 16-byte path) 159-161 us, 4 x 8 at
// 168 registers (spilling) 166 us, 4 x 6 175 us, 8 x 7 190 us; 4x4 with 8
// waves x 8 positions 157 us, 8 x 6 or 4 x 12 174-176 us, 8 x 10 184 us,
// 4 x 8 or 16 x 4 236-240 us.
constexpr BlkRowCfg kBlkRow8{4, 7, 3};
constexpr BlkRowCfg kBlkRow4{8, 8, 1};
// The lane exchanges of the lane-group scan ride on the multiply-adds
// (v_fmac_f32 with a DPP operand) instead of separate DPP moves.
constexpr bool kBlkRowDppFma = true;

// Workspace: header, then per chunk the aggregate rows (k + 1 words per
// row) and the inclusive state rows (one word), both [chunk][word][row].
struct BlkRowWs {
    int64_t T, ncb, nq, ntiles, nrow;
    size_t hdr, agg, inc, total;
};

inline BlkRowWs blkrow_ws(int k, int64_t B, int64_t L, int64_t H) {
    const BlkRowCfg cfg = k == 8 ? kBlkRow8 : kBlkRow4;
    BlkRowWs w;
    w.T = (int64_t)cfg.nw * cfg.c;
    const int64_t heads = 64 / k;
    w.ncb = (H + heads - 1) / heads;
    w.nq = (L + w.T - 1) / w.T;
    w.ntiles = w.nq * B * w.ncb;
    w.nrow = B * H * k;
    Carve c;
    w.hdr = c.take(16);
    w.agg = c.take((size_t)w.nq * (k + 1) * w.nrow * 8);
    w.inc = c.take((size_t)w.nq * w.nrow * 8);
    w.total = c.off;
    return w;
}

// Newton steps of the GRU with dense recurrence inside heads of k channels
// (hgru.hip): one launch per iteration on the lane-group scan.  Measured for
// k = 8 at B=16 L=2048 NH=64, 4 iterations, with a sub-chunk's loads issued
// before its cells: 4 waves x 6 positions (162 VGPRs, three waves per SIMD)
// 0.93 ms, 4 x 8 bounded to 168 registers (spilling) 0.92-0.93, 4 x 8 at 181
// registers 0.96, 2 x 8 1.01-1.03, 4 x 4 1.08, 8 x 8 1.10, 8 x 4 1.53.
constexpr BlkRowCfg kHgru8{4, 6, 3};
constexpr BlkRowCfg kHgru4{8, 4, 1};

// Workspace: header, a max|delta| slot per iteration and two sets of
// chunk-boundary states (kept across the launches of a call: [maxd,
// keep_end)), then the look-back records of one launch.
struct HgruWs {
    BlkRowWs sh;  // chunking and record layout (the sh.hdr/agg/inc/total offsets unused)
    size_t hdr, maxd, bnd[2], keep_end, agg, inc, total;
};

inline HgruWs hgru_ws(int k, int64_t B, int64_t L, int64_t NH, int32_t cap) {
    const BlkRowCfg cfg = k == 8 ? kHgru8 : kHgru4;
    HgruWs w;
    w.sh.T = (int64_t)cfg.nw * cfg.c;
    const int64_t heads = 64 / k;
    w.sh.ncb = (NH + heads - 1) / heads;
    w.sh.nq = (L + w.sh.T - 1) / w.sh.T;
    w.sh.ntiles = w.sh.nq * B * w.sh.ncb;
    w.sh.nrow = B * NH * k;
    Carve c;
    w.hdr = c.take(16);
    w.maxd = c.take((size_t)cap * 4);
    for (int i = 0; i < 2; ++i) w.bnd[i] = c.take((size_t)w.sh.nq * w.sh.nrow * 4);
    w.keep_end = c.off;
    w.agg = c.take((size_t)w.sh.nq * (k + 1) * w.sh.nrow * 8);
    w.inc = c.take((size_t)w.sh.nq * w.sh.nrow * 8);
    w.total = c.off;
    return w;
}

// Gradients of the head GRU (hgru.hip, the adjoint on the lane-group scan,
// positions in reverse time): each lane keeps its rows of dL/dUz, dL/dUr,
// dL/dUc over its positions; a workgroup sums them over its waves into one
// partial per (tile, head), and a second launch sums the partials of each
// head over chunks and batch rows.  Measured for k = 8 at B=16 L=2048
// NH=64: 4 waves x 8 positions (247 VGPRs) 372-376 us, 8 x 6 434, 4 x 6
// 435, 2 x 8 469-493, 8 x 4 525, 4 x 4 540, 4 x 6 bounded to 168 registers
// 567.
constexpr BlkRowCfg kHgruAdj8{4, 8, 1};
constexpr BlkRowCfg kHgruAdj4{8, 4, 1};

constexpr int kHgruUSlices = 64;  // slices of the first dL/dU reduction pass

struct HgruAdjWs {
    BlkRowWs sh;     // chunking and look-back records
    size_t partial;  // [tile][64/k heads][3 gates][k][k] floats (kept at a wrap clear)
    size_t stage;    // [NH][3][kHgruUSlices][k][k] floats, the first pass's sums
    size_t total;
};

inline HgruAdjWs hgru_adj_ws(int k, int64_t B, int64_t L, int64_t NH) {
    const BlkRowCfg cfg = k == 8 ? kHgruAdj8 : kHgruAdj4;
    HgruAdjWs w;
    w.sh.T = (int64_t)cfg.nw * cfg.c;
    const int64_t heads = 64 / k;
    w.sh.ncb = (NH + heads - 1) / heads;
    w.sh.nq = (L + w.sh.T - 1) / w.sh.T;
    w.sh.ntiles = w.sh.nq * B * w.sh.ncb;
    w.sh.nrow = B * NH * k;
    Carve c;
    w.sh.hdr = c.take(16);
    w.sh.agg = c.take((size_t)w.sh.nq * (k + 1) * w.sh.nrow * 8);
    w.sh.inc = c.take((size_t)w.sh.nq * w.sh.nrow * 8);
    w.partial = c.take((size_t)w.sh.ntiles * heads * 3 * k * k * 4);
    w.stage = c.take((size_t)NH * 3 * kHgruUSlices * k * k * 4);
    w.sh.total = w.total = c.off;
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
