// api.hip -- the C ABI declared in include/pararnn.h: host-side argument
// validation, workspace checks and dispatch to the kernel launchers.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "pararnn.h"
#include "launch.hpp"

using namespace prn;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 40;

bool dims_ok(int64_t B, int64_t L, int64_t H) {
    if (B <= 0 || L <= 0 || H <= 0) return false;
    if (B > kMaxDim || L > kMaxDim || H > kMaxDim) return false;
    // B*L*H elements must be addressable and the grid must fit in 2^31 blocks
    const double n = (double)B * (double)L * (double)H;
    return n < 9.0e15;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? PARARNN_OK : PARARNN_ERR_HIP; }

bool grid_ok(int64_t ntiles) { return ntiles > 0 && ntiles < ((int64_t)1 << 31); }

// Whether the n-float arrays at p and q share any byte (a null one shares none).
bool overlaps(const float *p, const float *q, int64_t n) {
    if (p == nullptr || q == nullptr) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q, len = (uintptr_t)n * sizeof(float);
    return a < b + len && b < a + len;
}

// Zeros for trace entries [from, to) that no iteration will write.
int clear_trace_tail(float *trace, int32_t from, int32_t to, hipStream_t s) {
    FillRange fr[1] = {{trace + from, (uint64_t)(to - from), 0, 4}};
    return status_of(fill(fr, 1, s));
}

// Newton from zero reproduces the sequential result after L iterations (and
// iteration L + 1 confirms it with a zero update), so caps above L + 1 change
// nothing but the number of launches: they are taken as L + 1 (a trace still
// receives zeros up to the caller's cap).
int32_t eff_cap(int32_t max_iter, int64_t L) {
    return (int64_t)max_iter > L + 1 ? (int32_t)(L + 1) : max_iter;
}

// The chained kernel keeps records of every iteration, so its workspace
// grows with the cap; above kChainMaxCap the per-iteration path is used.
bool chain_ok(int32_t cap) { return cap <= kChainMaxCap; }


// Path of a Newton forward.  The GRU takes the fused on-chip kernel while
// the sequence fits one workgroup's registers; longer sequences (and the
// LSTM) take the chained kernel, which keeps each chunk on chip for all its
// iterations, unless the cap is above kChainMaxCap.  The chained kernel lets
// each workgroup own whole chains of chunks when there are at least as many
// chains as workgroup slots, and chains chunks across workgroups otherwise.
// PARARNN_GRU_PATH=fused|chain|local|step and PARARNN_LSTM_PATH=chain|local|step
// override the choice (for testing every path; "chain" and "local" force the
// two forms of the chained kernel, "local" only with channel lanes; a chain
// request above kChainMaxCap still takes the per-iteration path).
enum class Path { Fused, Chain, Step, Invalid };
Path env_path(const char *name) {
    const char *env = getenv(name);
    if (env == nullptr) return Path::Invalid;
    if (strcmp(env, "fused") == 0) return Path::Fused;
    if (strcmp(env, "chain") == 0 || strcmp(env, "local") == 0) return Path::Chain;
    if (strcmp(env, "step") == 0) return Path::Step;
    return Path::Invalid;
}
// Form of the chained kernel: 1 workgroups own whole chains, 0 chunks are
// chained across workgroups, -1 chosen from the shape.
int env_chain_local(const char *name) {
    const char *env = getenv(name);
    if (env == nullptr) return -1;
    if (strcmp(env, "local") == 0) return 1;
    if (strcmp(env, "chain") == 0) return 0;
    return -1;
}
Path gru_path(int64_t L, int32_t cap) {
    const bool fits = fused_c_for(L) != 0;
    const Path p = env_path("PARARNN_GRU_PATH");
    if (p == Path::Fused) return fits ? Path::Fused : Path::Invalid;
    if (p == Path::Step) return p;
    if (p == Path::Chain) return chain_ok(cap) ? p : Path::Step;
    return fits ? Path::Fused : (chain_ok(cap) ? Path::Chain : Path::Step);
}
Path lstm_path(int32_t cap) {
    const Path p = env_path("PARARNN_LSTM_PATH");
    return (p == Path::Step || !chain_ok(cap)) ? Path::Step : Path::Chain;
}

// Workspace of a Newton forward: that of the kernel the call takes (the
// fused kernel and the chained kernel's whole-chain form use none; the query
// returns the 256-byte minimum for them).
constexpr size_t kMinWs = 256;
size_t gru_fwd_ws(int64_t B, int64_t L, int64_t H, int32_t cap) {
    switch (gru_path(L, cap)) {
        case Path::Chain:
            if (gru_chain_owns_chains(B, L, H, env_chain_local("PARARNN_GRU_PATH"))) return kMinWs;
            return chain_ws(kCfgGruChain, 1, B, L, H, cap).total;
        case Path::Step: return newton_ws(kCfgGruStep, 1, B, L, H, cap).total;
        default: return kMinWs;
    }
}
// The 4x4 blocks take the lane-group kernel (blkrow.hip) unless
// PARARNN_BLK4_PATH=thread asks for the one-thread-per-block scan.
bool blk4_rows() {
    const char *env = getenv("PARARNN_BLK4_PATH");
    return !(env != nullptr && strcmp(env, "thread") == 0);
}
size_t blk4_ws(int64_t B, int64_t L, int64_t H) {
    return blk4_rows() ? blkrow_ws(4, B, L, H).total : scan_ws(kCfgLinBlk4, 4, B, L, H).total;
}

size_t lstm_fwd_ws(int64_t B, int64_t L, int64_t H, int32_t cap) {
    if (lstm_path(cap) == Path::Step) return newton_ws(kCfgLstmStep, 2, B, L, H, cap).total;
    if (lstm_chain_owns_chains(B, L, H, env_chain_local("PARARNN_LSTM_PATH"))) return kMinWs;
    return chain_ws(kCfgLstmChain, 2, B, L, H, cap).total;
}

}  // namespace

extern "C" {

const char *pararnn_status_string(int status) {
    switch (status) {
        case PARARNN_OK: return "ok";
        case PARARNN_ERR_INVALID: return "invalid argument";
        case PARARNN_ERR_HIP: return "HIP error";
        case PARARNN_ERR_UNSUPPORTED: return "unsupported";
        case PARARNN_ERR_TOO_LARGE: return "needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

size_t pararnn_workspace_bytes(int32_t op, int64_t B, int64_t L, int64_t H, int32_t max_iter) {
    if (!dims_ok(B, L, H)) return 0;
    switch (op) {
        case PARARNN_OP_LINSCAN_DIAG: return scan_ws(kCfgLinDiag, 1, B, L, H).total;
        case PARARNN_OP_LINSCAN_BLK2: return scan_ws(kCfgLinBlk2, 2, B, L, H).total;
        case PARARNN_OP_GRU_FORWARD:
            if (max_iter < 1) return 0;
            return gru_fwd_ws(B, L, H, eff_cap(max_iter, L));
        case PARARNN_OP_LSTM_FORWARD:
            if (max_iter < 1) return 0;
            return lstm_fwd_ws(B, L, H, eff_cap(max_iter, L));
        case PARARNN_OP_LINSCAN_BLK4: return blk4_ws(B, L, H);
        case PARARNN_OP_LINSCAN_BLK8: return blkrow_ws(8, B, L, H).total;
        case PARARNN_OP_HGRU4_FORWARD:
        case PARARNN_OP_HGRU8_FORWARD: {
            const int k = op == PARARNN_OP_HGRU8_FORWARD ? 8 : 4;
            if (max_iter < 1 || !dims_ok(B, L, H * k)) return 0;
            return hgru_ws(k, B, L, H, eff_cap(max_iter, L)).total;
        }
        case PARARNN_OP_HGRU4_BACKWARD:
        case PARARNN_OP_HGRU8_BACKWARD: {
            const int k = op == PARARNN_OP_HGRU8_BACKWARD ? 8 : 4;
            if (!dims_ok(B, L, H * k)) return 0;
            return hgru_adj_ws(k, B, L, H).total;
        }
        case PARARNN_OP_GRU_ADJOINT: return gru_adjoint_ws(B, L, H);
        case PARARNN_OP_LSTM_ADJOINT: return lstm_adjoint_ws(B, L, H);
        default: return 0;
    }
}

int rnn_linscan_diag(int64_t B, int64_t L, int64_t H, const float *a, const float *b,
                     const float *h0, float *h, void *ws, size_t ws_bytes, void *stream) {
    if (!dims_ok(B, L, H) || !a || !b || !h || !ws) return PARARNN_ERR_INVALID;
    if (!grid_ok(scan_shape(kCfgLinDiag, B, L, H).ntiles)) return PARARNN_ERR_INVALID;
    if (ws_bytes < scan_ws(kCfgLinDiag, 1, B, L, H).total || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    return status_of(linscan_diag(B, L, H, a, b, h0, h, Ws{static_cast<char *>(ws), ws_bytes},
                                  static_cast<hipStream_t>(stream)));
}

int rnn_linscan_blk2(int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                     const float *h0, float *h, void *ws, size_t ws_bytes, void *stream) {
    if (!dims_ok(B, L, H) || !A || !b || !h || !ws) return PARARNN_ERR_INVALID;
    if (!aligned(A, 4) || !aligned(b, 4) || !aligned(h, 4) || (h0 && !aligned(h0, 4)))
        return PARARNN_ERR_INVALID;
    if (!grid_ok(scan_shape(kCfgLinBlk2, B, L, H).ntiles)) return PARARNN_ERR_INVALID;
    if (ws_bytes < scan_ws(kCfgLinBlk2, 2, B, L, H).total || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    return status_of(linscan_blk2(B, L, H, A, b, h0, h, Ws{static_cast<char *>(ws), ws_bytes},
                                  static_cast<hipStream_t>(stream)));
}

int rnn_linscan_blk(int32_t k, int64_t B, int64_t L, int64_t H, const float *A, const float *b,
                    const float *h0, float *h, void *ws, size_t ws_bytes, void *stream) {
    if (k == 2) return rnn_linscan_blk2(B, L, H, A, b, h0, h, ws, ws_bytes, stream);
    if (k < 1) return PARARNN_ERR_INVALID;
    if (k != 4 && k != 8) return PARARNN_ERR_UNSUPPORTED;
    if (!dims_ok(B, L, H) || !A || !b || !h || !ws) return PARARNN_ERR_INVALID;
    if (!aligned(A, 4) || !aligned(b, 4) || !aligned(h, 4) || (h0 && !aligned(h0, 4)))
        return PARARNN_ERR_INVALID;
    const Ws w{static_cast<char *>(ws), ws_bytes};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 4 && !blk4_rows()) {
        if (!grid_ok(scan_shape(kCfgLinBlk4, B, L, H).ntiles)) return PARARNN_ERR_INVALID;
        if (ws_bytes < scan_ws(kCfgLinBlk4, 4, B, L, H).total || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
        return status_of(linscan_blk(4, B, L, H, A, b, h0, h, w, s));
    }
    const BlkRowWs need = blkrow_ws(k, B, L, H);
    if (!grid_ok(need.ntiles)) return PARARNN_ERR_INVALID;
    if (ws_bytes < need.total || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    return status_of(linscan_blkrow(k, B, L, H, A, b, h0, h, w, s));
}

int pararnn_gru_forward(int64_t B, int64_t L, int64_t H, const float *pz, const float *pr,
                        const float *pc, const float *uz, const float *ur, const float *uc,
                        const float *h0, const float *h_init, float *h, float tol, int32_t max_iter,
                        int32_t *info, float *trace, void *ws, size_t ws_bytes, void *stream) {
    if (!dims_ok(B, L, H) || !pz || !pr || !pc || !uz || !ur || !uc || !h) return PARARNN_ERR_INVALID;
    if (!(tol >= 0.0f) || max_iter < 1) return PARARNN_ERR_INVALID;  // rejects NaN too
    if (overlaps(h_init, h, B * L * H)) return PARARNN_ERR_INVALID;
    const int32_t cap = eff_cap(max_iter, L);
    GruFwdArgs a{B,  L,   H,   pz,    pr,   pc,    uz,   ur,
                 uc, h0,  h_init, h,  tol,  cap,   info, trace,
                 env_chain_local("PARARNN_GRU_PATH")};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Path path = gru_path(L, cap);
    if (path == Path::Invalid) return PARARNN_ERR_UNSUPPORTED;
    if (path != Path::Fused && (!ws || ws_bytes < gru_fwd_ws(B, L, H, cap) || !aligned(ws, 256)))
        return PARARNN_ERR_INVALID;
    const int64_t ntiles = path == Path::Fused ? B * ((H + kFusedChannels - 1) / kFusedChannels)
                           : path == Path::Chain ? scan_shape(kCfgGruChain, B, L, H).ntiles
                                                 : scan_shape(kCfgGruStep, B, L, H).ntiles;
    if (!grid_ok(ntiles)) return PARARNN_ERR_INVALID;
    if (trace != nullptr && max_iter > cap) {
        const int st = clear_trace_tail(trace, cap, max_iter, s);
        if (st != PARARNN_OK) return st;
    }
    const Ws w{static_cast<char *>(ws), ws_bytes};
    if (path == Path::Fused) return status_of(gru_forward_fused(a, s));
    if (path == Path::Chain) return status_of(gru_forward_chain(a, w, s));
    return status_of(gru_forward_step(a, w, s));
}

int pararnn_lstm_forward(int64_t B, int64_t L, int64_t H, const float *pi, const float *pf,
                         const float *po, const float *pg, const float *ui, const float *uf,
                         const float *uo, const float *ug, const float *h0, const float *c0,
                         const float *h_init, const float *c_init, float *h, float *c, float tol,
                         int32_t max_iter, int32_t *info, float *trace, void *ws, size_t ws_bytes,
                         void *stream) {
    if (!dims_ok(B, L, H) || !pi || !pf || !po || !pg || !ui || !uf || !uo || !ug || !h || !c)
        return PARARNN_ERR_INVALID;
    if (!(tol >= 0.0f) || max_iter < 1) return PARARNN_ERR_INVALID;
    const int64_t n = B * L * H;
    if (overlaps(h_init, h, n) || overlaps(h_init, c, n) || overlaps(c_init, h, n) || overlaps(c_init, c, n))
        return PARARNN_ERR_INVALID;
    const int32_t cap = eff_cap(max_iter, L);
    if (!ws || ws_bytes < lstm_fwd_ws(B, L, H, cap) || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    LstmFwdArgs a{B,  L,  H,      pi,     pf, po, pg,  ui,  uf,   uo,    ug,
                  h0, c0, h_init, c_init, h,  c,  tol, cap, info, trace, env_chain_local("PARARNN_LSTM_PATH")};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool chain = lstm_path(cap) == Path::Chain;
    if (!grid_ok(scan_shape(chain ? kCfgLstmChain : kCfgLstmStep, B, L, H).ntiles)) return PARARNN_ERR_INVALID;
    if (trace != nullptr && max_iter > cap) {
        const int st = clear_trace_tail(trace, cap, max_iter, s);
        if (st != PARARNN_OK) return st;
    }
    const Ws w{static_cast<char *>(ws), ws_bytes};
    if (chain) return status_of(lstm_forward_chain(a, w, s));
    return status_of(lstm_forward_step(a, w, s));
}

int pararnn_hgru_forward(int32_t k, int64_t B, int64_t L, int64_t NH, const float *pz, const float *pr,
                         const float *pc, const float *Uz, const float *Ur, const float *Uc, const float *h0,
                         const float *h_init, float *h, float tol, int32_t max_iter, int32_t *info, float *trace,
                         void *ws, size_t ws_bytes, void *stream) {
    if (k < 1) return PARARNN_ERR_INVALID;
    if (k != 4 && k != 8) return PARARNN_ERR_UNSUPPORTED;
    if (!dims_ok(B, L, NH) || !dims_ok(B, L, NH * k)) return PARARNN_ERR_INVALID;
    if (!pz || !pr || !pc || !Uz || !Ur || !Uc || !h) return PARARNN_ERR_INVALID;
    if (!(tol >= 0.0f) || max_iter < 1) return PARARNN_ERR_INVALID;
    if (overlaps(h_init, h, B * L * NH * k)) return PARARNN_ERR_INVALID;
    const int32_t cap = eff_cap(max_iter, L);
    const HgruWs need = hgru_ws(k, B, L, NH, cap);
    if (!grid_ok(need.sh.ntiles)) return PARARNN_ERR_INVALID;
    if (!ws || ws_bytes < need.total || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (trace != nullptr && max_iter > cap) {
        const int st = clear_trace_tail(trace, cap, max_iter, s);
        if (st != PARARNN_OK) return st;
    }
    const HgruFwdArgs a{k, B, L, NH, pz, pr, pc, Uz, Ur, Uc, h0, h_init, h, tol, cap, info, trace};
    return status_of(hgru_forward(a, Ws{static_cast<char *>(ws), ws_bytes}, s));
}

int pararnn_hgru_backward(int32_t k, int64_t B, int64_t L, int64_t NH, const float *pz, const float *pr,
                          const float *pc, const float *Uz, const float *Ur, const float *Uc, const float *h0,
                          const float *h, const float *grad_h, float *grad_pz, float *grad_pr, float *grad_pc,
                          float *grad_Uz, float *grad_Ur, float *grad_Uc, float *grad_h0, void *ws,
                          size_t ws_bytes, void *stream) {
    if (k < 1) return PARARNN_ERR_INVALID;
    if (k != 4 && k != 8) return PARARNN_ERR_UNSUPPORTED;
    if (!dims_ok(B, L, NH) || !dims_ok(B, L, NH * k)) return PARARNN_ERR_INVALID;
    if (!pz || !pr || !pc || !Uz || !Ur || !Uc || !h || !grad_h || !grad_pz || !grad_pr || !grad_pc)
        return PARARNN_ERR_INVALID;
    const int64_t n = B * L * NH * k;
    // h is read at other positions than the thread's own: no output may alias it
    if (overlaps(grad_pz, h, n) || overlaps(grad_pr, h, n) || overlaps(grad_pc, h, n)) return PARARNN_ERR_INVALID;
    if ((grad_Uz || grad_Ur || grad_Uc) && NH > 0x7fffffff) return PARARNN_ERR_INVALID;
    const HgruAdjWs need = hgru_adj_ws(k, B, L, NH);
    if (!grid_ok(need.sh.ntiles)) return PARARNN_ERR_INVALID;
    if (!ws || ws_bytes < need.total || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    HgruBwdArgs a{k, B, L, NH, pz, pr, pc, Uz, Ur, Uc, h0, h, grad_h, grad_pz, grad_pr, grad_pc,
                  {grad_Uz, grad_Ur, grad_Uc}, grad_h0};
    return status_of(hgru_backward(a, Ws{static_cast<char *>(ws), ws_bytes}, static_cast<hipStream_t>(stream)));
}

int pararnn_gru_sequential(int64_t B, int64_t L, int64_t H, const float *pz, const float *pr,
                           const float *pc, const float *uz, const float *ur, const float *uc,
                           const float *h0, float *h, void *stream) {
    if (!dims_ok(B, L, H) || !pz || !pr || !pc || !uz || !ur || !uc || !h) return PARARNN_ERR_INVALID;
    if (!grid_ok((B * H + 63) / 64)) return PARARNN_ERR_INVALID;
    GruFwdArgs a{B, L, H, pz, pr, pc, uz, ur, uc, h0, nullptr, h, 0.0f, 1, nullptr, nullptr, -1};
    return status_of(gru_rollout(a, static_cast<hipStream_t>(stream)));
}

int pararnn_lstm_sequential(int64_t B, int64_t L, int64_t H, const float *pi, const float *pf,
                            const float *po, const float *pg, const float *ui, const float *uf,
                            const float *uo, const float *ug, const float *h0, const float *c0,
                            float *h, float *c, void *stream) {
    if (!dims_ok(B, L, H) || !pi || !pf || !po || !pg || !ui || !uf || !uo || !ug || !h || !c)
        return PARARNN_ERR_INVALID;
    if (!grid_ok((B * H + 63) / 64)) return PARARNN_ERR_INVALID;
    LstmFwdArgs a{B, L, H, pi, pf, po, pg, ui, uf, uo, ug, h0, c0, nullptr, nullptr, h, c, 0.0f, 1, nullptr, nullptr, -1};
    return status_of(lstm_rollout(a, static_cast<hipStream_t>(stream)));
}

int pararnn_adjoint_backward(int32_t cell, int64_t B, int64_t L, int64_t H, const float *const *p,
                             const float *const *u, const float *h0, const float *c0,
                             const float *h, const float *c, const float *grad_h,
                             const float *grad_c, float *const *grad_p, float *const *grad_u,
                             float *grad_h0, float *grad_c0, void *ws, size_t ws_bytes,
                             void *stream) {
    if (cell != PARARNN_CELL_GRU && cell != PARARNN_CELL_LSTM) return PARARNN_ERR_INVALID;
    if (!dims_ok(B, L, H) || !p || !u || !h || !grad_h || !grad_p || !ws) return PARARNN_ERR_INVALID;
    const int ng = cell == PARARNN_CELL_GRU ? 3 : 4;
    AdjArgs a;
    memset(&a, 0, sizeof(a));
    a.B = B;
    a.L = L;
    a.H = H;
    for (int q = 0; q < ng; ++q) {
        if (!p[q] || !u[q] || !grad_p[q]) return PARARNN_ERR_INVALID;
        a.p[q] = p[q];
        a.u[q] = u[q];
        a.gp[q] = grad_p[q];
        a.gu[q] = grad_u ? grad_u[q] : nullptr;
    }
    a.h0 = h0;
    a.h = h;
    a.gh = grad_h;
    a.gh0 = grad_h0;
    bool want_u = false;
    for (int q = 0; q < ng; ++q) want_u = want_u || a.gu[q] != nullptr;
    if (want_u && H > 0x7fffffff) return PARARNN_ERR_INVALID;  // the dL/du reduction has one workgroup per channel
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cell == PARARNN_CELL_GRU) {
        if (grad_c || grad_c0) return PARARNN_ERR_INVALID;
        if (!grid_ok(scan_shape(kCfgGruAdj, B, L, H).ntiles)) return PARARNN_ERR_INVALID;
        if (ws_bytes < gru_adjoint_ws(B, L, H) || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
        return status_of(gru_adjoint(a, Ws{static_cast<char *>(ws), ws_bytes}, s));
    }
    if (!c) return PARARNN_ERR_INVALID;
    a.c0 = c0;
    a.c = c;
    a.gc = grad_c;
    a.gc0 = grad_c0;
    if (!grid_ok(scan_shape(kCfgLstmAdj, B, L, H).ntiles)) return PARARNN_ERR_INVALID;
    if (ws_bytes < lstm_adjoint_ws(B, L, H) || !aligned(ws, 256)) return PARARNN_ERR_INVALID;
    return status_of(lstm_adjoint(a, Ws{static_cast<char *>(ws), ws_bytes}, s));
}

}  // extern "C"
