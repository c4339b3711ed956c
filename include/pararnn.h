/*
 * pararnn.h -- C ABI of libpararnn.so: parallel-in-time evaluation of
 * nonlinear RNNs by Newton's method with a parallel linear-recurrence scan,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (ParaRNN page, TL;DR and abstract; DEER summary page, first and
 * second paragraphs): the recurrence h_t = f(h_{t-1}, x_t) over a whole
 * sequence is one nonlinear system; Newton's method linearises every cell at
 * the current iterate and solves the resulting block bi-diagonal linear
 * system, which is a linear recurrence, with a parallel scan over the
 * sequence.  The GRU-style cell has a diagonal Jacobian and the LSTM-style
 * cell a 2x2 block-diagonal one (ParaRNN page, Fig. 2 caption).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are fp32, dense, row-major.  Sequence tensors are [B, L, H]
 *    with the channel index fastest ("channel-contiguous").  Per-channel
 *    weights u are [H], shared over batch and time.  Initial states are
 *    [B, H].  Output row t is the state after consuming input t; the initial
 *    state is not emitted.
 *  - Every pointer named as a tensor is a DEVICE pointer (hipMalloc'd or
 *    torch-allocated, at least 4-byte aligned).  The caller owns all memory,
 *    including the workspace; the library never allocates or frees and keeps
 *    no state of its own between calls beyond cached device properties (what
 *    persists lives in the caller's workspace).  Outputs must not alias
 *    inputs.
 *  - `ws`/`ws_bytes`: a device scratch buffer of at least
 *    pararnn_workspace_bytes(...) bytes (256-byte aligned); `ws_bytes` is
 *    its whole size.  It must be zero-filled before its first use
 *    (hipMemset, torch.zeros); every call leaves it ready for the next call
 *    of any entry point at any size that fits, so the caller never clears it
 *    again and must not write to it between calls.  Its first 16 bytes
 *    count the workgroups of a launch and number the launches; the
 *    look-back records of the scans carry the number of the launch that
 *    wrote them, which is why no call has to clear them.  Launch numbers
 *    repeat after 8,388,606 launches on one workspace: the launch that uses
 *    the last number clears all `ws_bytes` past the 16-byte header when its
 *    last workgroup finishes (about a millisecond per few hundred MB, once
 *    per period), so no record of an earlier period is ever read.
 *    Concurrent calls on different streams need different workspaces.  A
 *    workspace that was not zero-filled gives wrong results (the kernels
 *    still stay in bounds and finish).
 *  - `stream`: a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns; it never
 *    synchronises.  Device-side outputs (including `info`) are valid once
 *    the stream has been synchronised.
 *  - Return value: PARARNN_OK, or a negative status.  Argument validation is
 *    done on the host before anything is enqueued (PARARNN_ERR_INVALID).  A
 *    failed launch returns PARARNN_ERR_HIP.  Non-convergence of Newton is NOT
 *    an error: the outputs hold the last iterate and info reports it.
 */
#ifndef PARARNN_H
#define PARARNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PARARNN_OK = 0,
    PARARNN_ERR_INVALID = -1,     /* bad pointer, size, tolerance, cap or workspace */
    PARARNN_ERR_HIP = -2,         /* a HIP launch or runtime call failed */
    PARARNN_ERR_UNSUPPORTED = -3, /* combination not implemented */
    PARARNN_ERR_TOO_LARGE = -4    /* needs more than the library's static scratch buffer */
};

enum { PARARNN_CELL_GRU = 0, PARARNN_CELL_LSTM = 1 };

/* Operation codes for pararnn_workspace_bytes. */
enum {
    PARARNN_OP_LINSCAN_DIAG = 0,
    PARARNN_OP_LINSCAN_BLK2 = 1,
    PARARNN_OP_GRU_FORWARD = 2,
    PARARNN_OP_LSTM_FORWARD = 3,
    PARARNN_OP_GRU_ADJOINT = 4,
    PARARNN_OP_LSTM_ADJOINT = 5,
    PARARNN_OP_LINSCAN_BLK4 = 6,  /* rnn_linscan_blk with k = 4 */
    PARARNN_OP_LINSCAN_BLK8 = 7,  /* rnn_linscan_blk with k = 8 */
    PARARNN_OP_HGRU4_FORWARD = 8,  /* pararnn_hgru_forward with k = 4 (H = heads) */
    PARARNN_OP_HGRU8_FORWARD = 9,  /* pararnn_hgru_forward with k = 8 (H = heads) */
    PARARNN_OP_HGRU4_BACKWARD = 10, /* pararnn_hgru_backward with k = 4 (H = heads) */
    PARARNN_OP_HGRU8_BACKWARD = 11  /* pararnn_hgru_backward with k = 8 (H = heads) */
};

/*
 * Bytes of workspace that operation `op` needs at (B, L, H) with Newton
 * iteration cap `max_iter` (ignored by the scans and the adjoints).  For the
 * Newton forwards it is the need of the kernel the call will take, which
 * depends on the shape, the cap, the device (how many workgroups fit on it)
 * and the PARARNN_GRU_PATH / PARARNN_LSTM_PATH environment overrides as read
 * at the time of the query.  The GRU's fused kernel and the chained kernel's
 * form in which workgroups own whole chains need none: 256 bytes are
 * returned.  A call whose workspace is too small for its kernel returns
 * PARARNN_ERR_INVALID.  Returns 0 for invalid arguments.
 */
size_t pararnn_workspace_bytes(int32_t op, int64_t B, int64_t L, int64_t H,
                               int32_t max_iter);

/*
 * Diagonal linear recurrence, solved by a chunked parallel scan
 * (ParaRNN page, Fig. 2 left: the parallel reduction for diagonal systems;
 * DEER summary page: associative scan; minimal-RNN article: the recurrence a
 * parallel scan evaluates once gates do not depend on h):
 *     h[b,t,j] = a[b,t,j] * h[b,t-1,j] + b[b,t,j],   h[b,-1,j] = h0[b,j]
 * a, b, h: [B, L, H].  h0: [B, H], or NULL for zeros.
 */
int rnn_linscan_diag(int64_t B, int64_t L, int64_t H,
                     const float *a, const float *b, const float *h0,
                     float *h, void *ws, size_t ws_bytes, void *stream);

/*
 * 2x2 block linear recurrence (ParaRNN page, Fig. 2: the 2x2 block-diagonal
 * solver used by ParaLSTM):
 *     h[b,t,j,:] = A[b,t,j] @ h[b,t-1,j,:] + b[b,t,j,:]
 * A: [B, L, H, 2, 2] row-major blocks (a00, a01, a10, a11).
 * b, h: [B, L, H, 2].  h0: [B, H, 2] or NULL.  Any 4-byte alignment; with
 * A 16-byte aligned and b, h, h0 8-byte aligned, blocks and pairs move as
 * single vector accesses (faster).
 */
int rnn_linscan_blk2(int64_t B, int64_t L, int64_t H,
                     const float *A, const float *b, const float *h0,
                     float *h, void *ws, size_t ws_bytes, void *stream);

/*
 * k x k block linear recurrence: the 2x2 solver widened to small dense
 * blocks, such as the per-head Jacobians of a cell with dense recurrence
 * inside heads of k channels (ParaRNN page, Fig. 2 caption: block
 * bi-diagonal systems; DEER summary page, limitations paragraph: dense
 * Jacobians as the hidden size grows):
 *     h[b,t,j,:] = A[b,t,j] @ h[b,t-1,j,:] + b[b,t,j,:]
 * A: [B, L, H, k, k] row-major blocks (A[i][l] takes component l into i).
 * b, h: [B, L, H, k].  h0: [B, H, k] or NULL.
 * k = 2 is rnn_linscan_blk2 (its workspace query, PARARNN_OP_LINSCAN_BLK2).
 * k = 4 and k = 8 take the workspace of PARARNN_OP_LINSCAN_BLK4 and
 * PARARNN_OP_LINSCAN_BLK8 and any 4-byte alignment (with A 16-byte aligned,
 * block rows move as 16-byte accesses, faster).  The rows of each block are
 * spread over k lanes; PARARNN_BLK4_PATH=thread (read at the query and at
 * the call) makes k = 4 take the kernel with one thread per block instead.
 * Other k return PARARNN_ERR_UNSUPPORTED (k < 1: PARARNN_ERR_INVALID).
 */
int rnn_linscan_blk(int32_t k, int64_t B, int64_t L, int64_t H,
                    const float *A, const float *b, const float *h0,
                    float *h, void *ws, size_t ws_bytes, void *stream);

/*
 * GRU-style cell with diagonal recurrence (ParaGRU, ParaRNN page Fig. 2):
 *   z = sigmoid(pz + uz*h), r = sigmoid(pr + ur*h),
 *   c = tanh(pc + uc*(r*h)),  h' = (1 - z)*h + z*c
 * evaluated over the whole sequence by Newton's method (ParaRNN TL;DR;
 * DEER summary), from h = 0 or from a given initial iterate.
 * pz, pr, pc: [B, L, H] gate pre-projections (input projections and biases
 * already applied).  uz, ur, uc: [H].  h0: [B, H] or NULL.
 * h_init: [B, L, H] initial iterate (a warm start, such as the solution of a
 * nearby input), or NULL for zeros; read only, and it must not overlap h
 * (PARARNN_ERR_INVALID).  Newton from any iterate is exact after L
 * iterations, so the cap rule below holds for warm starts too; a start that
 * already solves the system returns after one iteration with a zero update.
 * h: [B, L, H] output.
 * tol >= 0: Newton stops once max|delta| <= tol (the only extra
 * hyper-parameter; DEER summary, second paragraph), measured after the
 * update and absolute.  Where the test is taken depends on the kernel:
 *  - L <= 512: over the whole sequence of each 16 channels of a batch row;
 *  - longer sequences with max_iter <= 64: each chunk of the sequence stops
 *    once it and every earlier chunk of its channels meet the bound, so the
 *    last chunk stops exactly when Newton over the whole sequence of those
 *    channels would (earlier chunks may freeze a few iterations sooner, with
 *    corrections of order tol^2 left);
 *  - max_iter > 64: over the whole tensor (one launch per iteration).
 * With tol = 0 nothing stops before the cap.  max_iter >= 1; caps above
 * L + 1 are taken as L + 1 (Newton from zero is exact after L iterations,
 * and iteration L + 1 confirms it).
 * info: device int32[2] {iterations, converged} or NULL.  iterations is the
 * largest number of updates any tile applied; converged is 1 only if every
 * tile met the tolerance.
 * trace: device float[max_iter] or NULL; receives max|delta| of each
 * iteration (0 for iterations not run).
 */
int pararnn_gru_forward(int64_t B, int64_t L, int64_t H,
                        const float *pz, const float *pr, const float *pc,
                        const float *uz, const float *ur, const float *uc,
                        const float *h0, const float *h_init, float *h, float tol,
                        int32_t max_iter, int32_t *info, float *trace,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * LSTM-style cell with diagonal recurrence (ParaLSTM, ParaRNN page Fig. 2):
 * per channel the state is (c, h) and the Jacobian a 2x2 block.
 *   i = sigmoid(pi + ui*h'), f = sigmoid(pf + uf*h'), o = sigmoid(po + uo*h'),
 *   g = tanh(pg + ug*h'),  c = f*c' + i*g,  h = o*tanh(c)
 * Newton from (c, h) = 0, or from the initial iterates h_init, c_init
 * ([B, L, H] each, a NULL one taken as zeros; read only, neither may overlap
 * h or c); max|delta| is taken over both components.
 * pi, pf, po, pg: [B, L, H]; ui, uf, uo, ug: [H]; h0, c0: [B, H] or NULL;
 * h, c: [B, L, H] outputs.  tol, max_iter, info, trace as for the GRU,
 * except that this cell has no single-tile kernel: the chunk rule applies at
 * every L when max_iter <= 64.
 */
int pararnn_lstm_forward(int64_t B, int64_t L, int64_t H,
                         const float *pi, const float *pf, const float *po,
                         const float *pg, const float *ui, const float *uf,
                         const float *uo, const float *ug, const float *h0,
                         const float *c0, const float *h_init, const float *c_init,
                         float *h, float *c, float tol, int32_t max_iter,
                         int32_t *info, float *trace,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * GRU with dense recurrence inside heads of k channels (k = 4 or 8): the
 * GRU-style cell above with each weight vector replaced by one k x k matrix
 * per head, acting on the state vector of the head where the diagonal cell
 * multiplies by u (a diagonal U is exactly the diagonal cell), so the
 * Jacobian is block-diagonal with dense k x k blocks (DEER summary page,
 * limitations paragraph: dense Jacobians, the GRU with 8-channel heads;
 * ParaRNN page, Fig. 2 caption: block bi-diagonal systems):
 *   z = sigmoid(pz + Uz h), r = sigmoid(pr + Ur h),
 *   c = tanh(pc + Uc (r*h)),  h' = (1 - z)*h + z*c
 * evaluated over the whole sequence by Newton's method, one launch per
 * iteration (launches after convergence exit at once; the host never waits),
 * each solving the block bi-diagonal system with the k x k scan.
 * pz, pr, pc: [B, L, NH, k] gate pre-projections; Uz, Ur, Uc: [NH, k, k]
 * row-major (U[n][i][l] takes component l into i); h0: [B, NH, k] or NULL;
 * h_init: [B, L, NH, k] initial iterate or NULL for zeros (must not overlap
 * h); h: [B, L, NH, k] output.  tol, max_iter, info, trace as for
 * pararnn_gru_forward, with max|delta| over the whole tensor (every cap
 * takes this path).  Workspace: PARARNN_OP_HGRU4_FORWARD /
 * PARARNN_OP_HGRU8_FORWARD with H = NH.  Other k return
 * PARARNN_ERR_UNSUPPORTED (k < 1: PARARNN_ERR_INVALID).
 */
int pararnn_hgru_forward(int32_t k, int64_t B, int64_t L, int64_t NH,
                         const float *pz, const float *pr, const float *pc,
                         const float *Uz, const float *Ur, const float *Uc,
                         const float *h0, const float *h_init, float *h, float tol,
                         int32_t max_iter, int32_t *info, float *trace,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Gradients through the converged solve of pararnn_hgru_forward (DEER
 * summary page: forward plus gradients; the adjoint is the transposed block
 * bi-diagonal system, ParaRNN page, Fig. 2 caption), by a reverse-time scan
 * of k x k blocks:
 *   nu_t = J_t^T (nu_{t+1} + g_t) with nu_L = 0,  lambda_t = g_t + nu_{t+1},
 *   dL/dpz = lambda dF/daz,  dL/dpc = lambda dF/dac,  dL/dpr = dL/dar,
 *   dL/dU = sum over batch rows and positions of the outer products of the
 *   pre-activation gradients with the vectors U multiplies (h for Uz and Ur,
 *   r*h for Uc),  dL/dh0 = nu_0,
 * for L = sum g*h, with the cell and J_t evaluated at the given states.
 * pz, pr, pc, Uz, Ur, Uc, h0 as for pararnn_hgru_forward; h: [B, L, NH, k]
 * the forward's solution; grad_h: [B, L, NH, k].  grad_pz, grad_pr,
 * grad_pc: [B, L, NH, k] outputs (overwritten; each may be its own p, none
 * may overlap h).  grad_Uz, grad_Ur, grad_Uc: [NH, k, k] outputs or NULL
 * (any of them requires NH < 2^31).  grad_h0: [B, NH, k] output or NULL.
 * Workspace: PARARNN_OP_HGRU4_BACKWARD / PARARNN_OP_HGRU8_BACKWARD with
 * H = NH (max_iter ignored).  Other k return PARARNN_ERR_UNSUPPORTED (k < 1:
 * PARARNN_ERR_INVALID).
 */
int pararnn_hgru_backward(int32_t k, int64_t B, int64_t L, int64_t NH,
                          const float *pz, const float *pr, const float *pc,
                          const float *Uz, const float *Ur, const float *Uc,
                          const float *h0, const float *h, const float *grad_h,
                          float *grad_pz, float *grad_pr, float *grad_pc,
                          float *grad_Uz, float *grad_Ur, float *grad_Uc, float *grad_h0,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Gradients through the converged solve (DEER summary: forward plus
 * gradients), by a reverse-time linear scan of the adjoint:
 *   lambda_t = g_t + J_{t+1}^T lambda_{t+1},  dL/dp_t = (df_t/dp_t)^T lambda_t,
 *   dL/du = sum_{b,t} lambda_t^T df_t/du,  dL/dh0 = J_0^T lambda_0,
 * for the loss L = sum g_h*h (+ sum g_c*c for the LSTM), with J and df/dp
 * evaluated at the forward states (h, c).
 * cell: PARARNN_CELL_GRU (3 gates z, r, c) or PARARNN_CELL_LSTM (4 gates
 * i, f, o, g).  p, u, grad_p, grad_u: HOST arrays of 3 or 4 DEVICE pointers.
 * h (and c for the LSTM): the forward outputs [B, L, H].  grad_h: [B, L, H];
 * grad_c: [B, L, H] or NULL (LSTM only; NULL means zero).  grad_p[k]:
 * [B, L, H] outputs (overwritten).  grad_u: NULL, or an array whose entries
 * are [H] outputs or NULL (any of them requires H < 2^31).  grad_h0,
 * grad_c0: [B, H] outputs or NULL.
 */
int pararnn_adjoint_backward(int32_t cell, int64_t B, int64_t L, int64_t H,
                             const float *const *p, const float *const *u,
                             const float *h0, const float *c0,
                             const float *h, const float *c,
                             const float *grad_h, const float *grad_c,
                             float *const *grad_p, float *const *grad_u,
                             float *grad_h0, float *grad_c0,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * Sequential application of the GRU-style cell: one thread per channel
 * walks t = 0..L-1 in order, one cell evaluation per position, no Newton
 * iteration.  This is the evaluation the pages quote their speedups against
 * (ParaRNN page, abstract and Fig. 2 caption: speedup over sequential
 * application; DEER summary page, results: sequential GRU at L = 2^20), and
 * the exact answer Newton converges to.  It exposes only B*H-fold
 * parallelism.  Arguments, layouts and the cell as for pararnn_gru_forward
 * (no tolerance, cap, info, trace or workspace).
 */
int pararnn_gru_sequential(int64_t B, int64_t L, int64_t H,
                           const float *pz, const float *pr, const float *pc,
                           const float *uz, const float *ur, const float *uc,
                           const float *h0, float *h, void *stream);

/*
 * Sequential application of the LSTM-style cell (as above; arguments as for
 * pararnn_lstm_forward without tolerance, cap, info, trace or workspace).
 */
int pararnn_lstm_sequential(int64_t B, int64_t L, int64_t H,
                            const float *pi, const float *pf, const float *po,
                            const float *pg, const float *ui, const float *uf,
                            const float *uo, const float *ug, const float *h0,
                            const float *c0, float *h, float *c, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the GRU
 * Newton forward of pararnn_gru_forward from h = 0 (no initial iterate),
 * with its other arguments, results and errors, but no workspace argument.  Its workspace is a static device
 * array of the library, PARARNN_NOALLOC_SCRATCH_BYTES bytes on each device
 * it runs on, held until the process ends.  The first call on a device looks
 * up the array's address (with that device current) and zero-fills it with
 * one kernel on `stream`; no call allocates or frees anything.  A shape
 * whose workspace (pararnn_workspace_bytes(PARARNN_OP_GRU_FORWARD, ...))
 * exceeds the array returns PARARNN_ERR_TOO_LARGE before anything is
 * enqueued.  Every call on a device shares the one array: calls that overlap
 * in time on one device (other streams, other threads) race on it and must
 * not be issued; consecutive calls, in any order of shapes, are fine.
 * The device is the current one, which must be the device of `stream`.
 */
#define PARARNN_NOALLOC_SCRATCH_BYTES (64u << 20)
int pararnn_gru_forward_noalloc(int64_t B, int64_t L, int64_t H,
                                const float *pz, const float *pr, const float *pc,
                                const float *uz, const float *ur, const float *uc,
                                const float *h0, float *h, float tol, int32_t max_iter,
                                int32_t *info, float *trace, void *stream);

/* Short text for a status code (static storage). */
const char *pararnn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PARARNN_H */
