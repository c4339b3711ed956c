/*
 * oracle.c -- plain, slow, obviously correct fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source with the GPU library.
 *
 * What it computes (sources on the pages):
 *  - The sequential application h[t] = f(h[t-1], x[t]) that defines the
 *    result (tutorial "The Parallelization Problem: Why GPUs Hated RNNs",
 *    code listing "Sequential vs parallel"; ParaRNN Fig. 5 caption,
 *    "sequential" modality; DEER summary: outputs agree with sequential
 *    evaluation).
 *  - Newton's method on the whole-sequence system h_t - f(h_{t-1}) = 0
 *    (ParaRNN TL;DR and abstract; DEER summary, first paragraph), each
 *    iteration solving the bi-diagonal linearised system by a serial
 *    forward substitution (ParaRNN TL;DR: block bi-diagonal system).
 *  - The diagonal (ParaGRU) and 2x2 block-diagonal (ParaLSTM) Jacobians
 *    (ParaRNN Fig. 2 caption).  The cell equations themselves are not printed
 *    on the pages; the GRU and LSTM cells below are the diagonal-recurrence
 *    forms of the classical cells that those captions name.
 *  - Gradients of L = sum g*h through the rollout, by plain reverse-mode
 *    backpropagation through time (DEER summary: forward plus gradients).
 *  - A GRU with dense recurrence inside heads of k channels (DEER summary,
 *    limitations paragraph): its rollout, Newton with k x k block Jacobians
 *    and backpropagation through time.
 *  - The linear recurrence h_t = a_t*h_{t-1} + b_t by a serial loop
 *    (minimal-RNN article: gates without h-dependence give a recurrence that
 *    a parallel scan solves; DEER summary: associative scan), and its 2x2 and
 *    k x k block forms (at most 8x8 here).
 *
 * All arithmetic is fp64 and in the natural sequential order.  Channels
 * (b, j) are independent and are spread over threads with OpenMP; that does
 * not change any result.
 *
 * Layout: sequence tensors [B, L, H] row-major (j fastest); blocks
 * [B, L, H, 2, 2] and pairs [B, L, H, 2]; weights u [H]; initial states [B, H].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IDX(b, t, j) (((size_t)(b) * (size_t)L + (size_t)(t)) * (size_t)H + (size_t)(j))

static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

/* -------------------------------------------------------------------------
 * GRU cell with diagonal recurrent weights (ParaGRU: diagonal Jacobian).
 *   z = sig(pz + uz*h), r = sig(pr + ur*h), c = tanh(pc + uc*(r*h)),
 *   f = (1 - z)*h + z*c.
 * Outputs f; optionally J = df/dh and the partials df/dp (pz, pr, pc).
 * The partials are obtained by the chain rule term by term.
 * ------------------------------------------------------------------------- */
void orc_gru_cell(double h, double pz, double pr, double pc,
                  double uz, double ur, double uc,
                  double *f, double *J, double *dfdp /* [3] or NULL */,
                  double *gates /* [3] = z, r, c or NULL */)
{
    double z = sigm(pz + uz * h);
    double r = sigm(pr + ur * h);
    double s = r * h;
    double c = tanh(pc + uc * s);
    *f = (1.0 - z) * h + z * c;

    double dz = z * (1.0 - z);      /* sigma'(.) */
    double dr = r * (1.0 - r);
    double dc = 1.0 - c * c;        /* tanh'(.) */
    if (J) {
        /* d/dh of (1-z)h:  (1-z) - h*dz/dh ;  d/dh of z*c:  c*dz/dh + z*dc/dh */
        double dz_dh = dz * uz;
        double ds_dh = r + h * dr * ur;
        double dc_dh = dc * uc * ds_dh;
        *J = (1.0 - z) - h * dz_dh + c * dz_dh + z * dc_dh;
    }
    if (dfdp) {
        dfdp[0] = (c - h) * dz;              /* df/dpz */
        dfdp[1] = z * dc * uc * h * dr;      /* df/dpr */
        dfdp[2] = z * dc;                    /* df/dpc */
    }
    if (gates) { gates[0] = z; gates[1] = r; gates[2] = c; }
}

/* -------------------------------------------------------------------------
 * LSTM cell with diagonal recurrent weights (ParaLSTM: 2x2 block Jacobian on
 * the per-channel state (c, h)).
 *   i = sig(pi + ui*h'), f = sig(pf + uf*h'), o = sig(po + uo*h'),
 *   g = tanh(pg + ug*h'), c = f*c' + i*g, h = o*tanh(c).
 * Outputs (c, h); optionally J (row-major: dc/dc', dc/dh', dh/dc', dh/dh')
 * and dcdp[4], dhdp[4] in gate order (i, f, o, g).
 * ------------------------------------------------------------------------- */
void orc_lstm_cell(double cp, double hp,
                   double pi, double pf, double po, double pg,
                   double ui, double uf, double uo, double ug,
                   double *c_out, double *h_out, double *J /* [4] */,
                   double *dcdp /* [4] */, double *dhdp /* [4] */)
{
    double i = sigm(pi + ui * hp);
    double f = sigm(pf + uf * hp);
    double o = sigm(po + uo * hp);
    double g = tanh(pg + ug * hp);
    double c = f * cp + i * g;
    double tc = tanh(c);
    double h = o * tc;
    *c_out = c;
    *h_out = h;

    double di = i * (1.0 - i), df = f * (1.0 - f), dO = o * (1.0 - o);
    double dg = 1.0 - g * g, dtc = 1.0 - tc * tc;
    if (J) {
        /* c depends on h' through i, f and g. */
        double dc_dhp = cp * df * uf + g * di * ui + i * dg * ug;
        double dc_dcp = f;
        J[0] = dc_dcp;
        J[1] = dc_dhp;
        /* h = o(h') * tanh(c(c', h')) */
        J[2] = o * dtc * dc_dcp;
        J[3] = dO * uo * tc + o * dtc * dc_dhp;
    }
    if (dcdp && dhdp) {
        dcdp[0] = g * di;      /* i */
        dcdp[1] = cp * df;     /* f */
        dcdp[2] = 0.0;         /* o */
        dcdp[3] = i * dg;      /* g */
        dhdp[0] = o * dtc * dcdp[0];
        dhdp[1] = o * dtc * dcdp[1];
        dhdp[2] = dO * tc;
        dhdp[3] = o * dtc * dcdp[3];
    }
}

/* -------------------------------------------------------------------------
 * Linear recurrences, serial loop.
 * diag:  h_t = a_t * h_{t-1} + b_t,       h_{-1} = h0 (NULL means 0)
 * blk2:  h_t = A_t h_{t-1} + b_t (2x2),   A row-major [a00 a01 a10 a11]
 * ------------------------------------------------------------------------- */
void orc_linscan_diag(int64_t B, int64_t L, int64_t H, const double *a,
                      const double *b, const double *h0, double *h)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double x = h0 ? h0[bb * H + j] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                size_t k = IDX(bb, t, j);
                x = a[k] * x + b[k];
                h[k] = x;
            }
        }
}

void orc_linscan_blk2(int64_t B, int64_t L, int64_t H, const double *A,
                      const double *b, const double *h0, double *h)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double x0 = h0 ? h0[(bb * H + j) * 2 + 0] : 0.0;
            double x1 = h0 ? h0[(bb * H + j) * 2 + 1] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                size_t k = IDX(bb, t, j);
                const double *M = A + 4 * k;
                double y0 = M[0] * x0 + M[1] * x1 + b[2 * k + 0];
                double y1 = M[2] * x0 + M[3] * x1 + b[2 * k + 1];
                x0 = y0;
                x1 = y1;
                h[2 * k + 0] = x0;
                h[2 * k + 1] = x1;
            }
        }
}

/* -------------------------------------------------------------------------
 * k x k block linear recurrence, serial loop (ParaRNN Fig. 2 caption: block
 * bi-diagonal systems whose blocks are the per-channel Jacobians, 2x2 for
 * ParaLSTM; DEER summary, limitations paragraph: dense Jacobians as the
 * hidden size grows).  Per (batch, channel) block:
 *     h_t = A_t h_{t-1} + b_t,   h_{-1} = h0 (NULL means 0)
 * A [B, L, H, k, k] row-major (A[i][l] multiplies component l into i),
 * b, h [B, L, H, k], h0 [B, H, k].
 * ------------------------------------------------------------------------- */
void orc_linscan_blk(int64_t k, int64_t B, int64_t L, int64_t H, const double *A,
                     const double *b, const double *h0, double *h)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double x[64], y[64];
            for (int64_t i = 0; i < k; ++i) x[i] = h0 ? h0[(bb * H + j) * k + i] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                size_t e = IDX(bb, t, j);
                const double *M = A + (size_t)k * k * e;
                for (int64_t i = 0; i < k; ++i) {
                    double acc = 0.0;
                    for (int64_t l = 0; l < k; ++l) acc += M[i * k + l] * x[l];
                    y[i] = acc + b[(size_t)k * e + i];
                }
                for (int64_t i = 0; i < k; ++i) {
                    x[i] = y[i];
                    h[(size_t)k * e + i] = x[i];
                }
            }
        }
}

/* -------------------------------------------------------------------------
 * Sequential rollouts: the definition of the result.
 * Output row t is the state after consuming input t; h0 is not emitted.
 * ------------------------------------------------------------------------- */
void orc_gru_rollout(int64_t B, int64_t L, int64_t H,
                     const double *pz, const double *pr, const double *pc,
                     const double *uz, const double *ur, const double *uc,
                     const double *h0, double *h)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double x = h0 ? h0[bb * H + j] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                size_t k = IDX(bb, t, j);
                double f;
                orc_gru_cell(x, pz[k], pr[k], pc[k], uz[j], ur[j], uc[j], &f,
                             NULL, NULL, NULL);
                x = f;
                h[k] = x;
            }
        }
}

void orc_lstm_rollout(int64_t B, int64_t L, int64_t H,
                      const double *pi, const double *pf, const double *po,
                      const double *pg, const double *ui, const double *uf,
                      const double *uo, const double *ug, const double *h0,
                      const double *c0, double *h, double *c)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double hx = h0 ? h0[bb * H + j] : 0.0;
            double cx = c0 ? c0[bb * H + j] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                size_t k = IDX(bb, t, j);
                double cn, hn;
                orc_lstm_cell(cx, hx, pi[k], pf[k], po[k], pg[k], ui[j], uf[j],
                              uo[j], ug[j], &cn, &hn, NULL, NULL, NULL);
                cx = cn;
                hx = hn;
                h[k] = hx;
                c[k] = cx;
            }
        }
}

/* -------------------------------------------------------------------------
 * Newton's method on the whole-sequence system (ParaRNN TL;DR and abstract;
 * DEER summary).  Unknowns s_0..s_{L-1}; equations s_t - f(s_{t-1}, p_t) = 0
 * with s_{-1} = initial state (fixed).  Start from s^0 = 0 everywhere.
 * Iteration k:
 *   F_t = f(s^{k-1}_{t-1}),  J_t = df/ds at s^{k-1}_{t-1},
 *   r_t = s^{k-1}_t - F_t,
 *   solve the bi-diagonal system  delta_t - J_t delta_{t-1} = -r_t,
 *   delta_{-1} = 0, by forward substitution,
 *   s^k = s^{k-1} + delta,  e_k = max |delta| over everything (NaN counts
 *   as +inf); stop when e_k <= tol or k = cap.
 * Returns the number of iterations applied; *converged is 1 when the last
 * e_k <= tol.  trace (length cap, may be NULL) receives e_1..e_iters.
 * s_init (may be NULL) replaces the zero start: the same iteration from a
 * given whole-sequence iterate s^0 (a warm start); iterate n from s^0 = the
 * k-th iterate from zero is the (k+n)-th iterate from zero.
 * ------------------------------------------------------------------------- */
static double absmax_update(double m, double d)
{
    if (isnan(d)) return INFINITY;
    double a = fabs(d);
    return a > m ? a : m;
}

int orc_gru_newton(int64_t B, int64_t L, int64_t H,
                   const double *pz, const double *pr, const double *pc,
                   const double *uz, const double *ur, const double *uc,
                   const double *h0, const double *s_init, double tol, int cap,
                   double *s, int *converged, double *trace)
{
    size_t N = (size_t)B * (size_t)L * (size_t)H;
    double *F = (double *)malloc(N * sizeof(double));
    double *Jm = (double *)malloc(N * sizeof(double));
    if (s_init)
        memcpy(s, s_init, N * sizeof(double));
    else
        memset(s, 0, N * sizeof(double));
    *converged = 0;
    int k;
    for (k = 1; k <= cap; ++k) {
        double e = 0.0;
#pragma omp parallel for collapse(2) schedule(static) reduction(max : e)
        for (int64_t bb = 0; bb < B; ++bb)
            for (int64_t j = 0; j < H; ++j) {
                /* assemble F_t and J_t at the previous iterate */
                for (int64_t t = 0; t < L; ++t) {
                    size_t kk = IDX(bb, t, j);
                    double prev = t == 0 ? (h0 ? h0[bb * H + j] : 0.0) : s[IDX(bb, t - 1, j)];
                    orc_gru_cell(prev, pz[kk], pr[kk], pc[kk], uz[j], ur[j],
                                 uc[j], &F[kk], &Jm[kk], NULL, NULL);
                }
                /* forward substitution for delta, then the update */
                double d = 0.0, em = 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    size_t kk = IDX(bb, t, j);
                    double r = s[kk] - F[kk];
                    d = Jm[kk] * d - r;
                    em = absmax_update(em, d);
                    /* s[kk] is read above before being overwritten; s_{t-1}
                       of the previous iterate was already consumed in the
                       assembly loop. */
                    s[kk] = s[kk] + d;
                }
                if (em > e) e = em;
            }
        if (trace) trace[k - 1] = e;
        if (e <= tol) {
            *converged = 1;
            break;
        }
    }
    free(F);
    free(Jm);
    return k > cap ? cap : k;
}

int orc_lstm_newton(int64_t B, int64_t L, int64_t H,
                    const double *pi, const double *pf, const double *po,
                    const double *pg, const double *ui, const double *uf,
                    const double *uo, const double *ug, const double *h0,
                    const double *c0, const double *h_init, const double *c_init,
                    double tol, int cap, double *h, double *c,
                    int *converged, double *trace)
{
    size_t N = (size_t)B * (size_t)L * (size_t)H;
    double *Fc = (double *)malloc(N * sizeof(double));
    double *Fh = (double *)malloc(N * sizeof(double));
    double *Jm = (double *)malloc(4 * N * sizeof(double));
    /* initial iterate: the given (h, c) trajectories, zero where NULL */
    if (h_init)
        memcpy(h, h_init, N * sizeof(double));
    else
        memset(h, 0, N * sizeof(double));
    if (c_init)
        memcpy(c, c_init, N * sizeof(double));
    else
        memset(c, 0, N * sizeof(double));
    *converged = 0;
    int k;
    for (k = 1; k <= cap; ++k) {
        double e = 0.0;
#pragma omp parallel for collapse(2) schedule(static) reduction(max : e)
        for (int64_t bb = 0; bb < B; ++bb)
            for (int64_t j = 0; j < H; ++j) {
                for (int64_t t = 0; t < L; ++t) {
                    size_t kk = IDX(bb, t, j);
                    double hp = t == 0 ? (h0 ? h0[bb * H + j] : 0.0) : h[IDX(bb, t - 1, j)];
                    double cp = t == 0 ? (c0 ? c0[bb * H + j] : 0.0) : c[IDX(bb, t - 1, j)];
                    orc_lstm_cell(cp, hp, pi[kk], pf[kk], po[kk], pg[kk], ui[j],
                                  uf[j], uo[j], ug[j], &Fc[kk], &Fh[kk],
                                  &Jm[4 * kk], NULL, NULL);
                }
                double dc = 0.0, dh = 0.0, em = 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    size_t kk = IDX(bb, t, j);
                    const double *M = &Jm[4 * kk];
                    double rc = c[kk] - Fc[kk];
                    double rh = h[kk] - Fh[kk];
                    double ndc = M[0] * dc + M[1] * dh - rc;
                    double ndh = M[2] * dc + M[3] * dh - rh;
                    dc = ndc;
                    dh = ndh;
                    em = absmax_update(em, dc);
                    em = absmax_update(em, dh);
                    c[kk] += dc;
                    h[kk] += dh;
                }
                if (em > e) e = em;
            }
        if (trace) trace[k - 1] = e;
        if (e <= tol) {
            *converged = 1;
            break;
        }
    }
    free(Fc);
    free(Fh);
    free(Jm);
    return k > cap ? cap : k;
}

/* -------------------------------------------------------------------------
 * Backpropagation through time for L = sum_t g_t * h_t (+ sum gc_t * c_t for
 * the LSTM), given the forward states.  Plain reverse loop over t with a
 * carried adjoint lambda:
 *   lambda_t = g_t + (J_{t+1})^T lambda_{t+1}
 *   dL/dp_t  = (df_t/dp_t)^T lambda_t
 *   dL/du   += dL/dp_t * (d pre-activation / d u)
 *   dL/dh0   = (J_0)^T lambda_0
 * Outputs may be NULL where not wanted (du, dh0, dc0).  du is accumulated
 * over b and t and is written, not added to.
 * ------------------------------------------------------------------------- */
void orc_gru_bptt(int64_t B, int64_t L, int64_t H,
                  const double *pz, const double *pr, const double *pc,
                  const double *uz, const double *ur, const double *uc,
                  const double *h0, const double *h, const double *g,
                  double *dpz, double *dpr, double *dpc,
                  double *duz, double *dur, double *duc, double *dh0)
{
    double *acc = (double *)calloc((size_t)B * (size_t)H * 3, sizeof(double));
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double lam = 0.0; /* adjoint carried from t+1 */
            double sz = 0.0, sr = 0.0, sc = 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                size_t kk = IDX(bb, t, j);
                lam += g[kk];
                double prev = t == 0 ? (h0 ? h0[bb * H + j] : 0.0) : h[IDX(bb, t - 1, j)];
                double f, J, dp[3], gt[3];
                orc_gru_cell(prev, pz[kk], pr[kk], pc[kk], uz[j], ur[j], uc[j],
                             &f, &J, dp, gt);
                dpz[kk] = dp[0] * lam;
                dpr[kk] = dp[1] * lam;
                dpc[kk] = dp[2] * lam;
                /* pre-activations: pz+uz*h', pr+ur*h', pc+uc*(r*h') */
                sz += dpz[kk] * prev;
                sr += dpr[kk] * prev;
                sc += dpc[kk] * gt[1] * prev;
                lam = J * lam;
            }
            if (dh0) dh0[bb * H + j] = lam;
            acc[(bb * H + j) * 3 + 0] = sz;
            acc[(bb * H + j) * 3 + 1] = sr;
            acc[(bb * H + j) * 3 + 2] = sc;
        }
    for (int64_t j = 0; j < H; ++j) {
        double a0 = 0, a1 = 0, a2 = 0;
        for (int64_t bb = 0; bb < B; ++bb) {
            a0 += acc[(bb * H + j) * 3 + 0];
            a1 += acc[(bb * H + j) * 3 + 1];
            a2 += acc[(bb * H + j) * 3 + 2];
        }
        if (duz) duz[j] = a0;
        if (dur) dur[j] = a1;
        if (duc) duc[j] = a2;
    }
    free(acc);
}

void orc_lstm_bptt(int64_t B, int64_t L, int64_t H,
                   const double *pi, const double *pf, const double *po,
                   const double *pg, const double *ui, const double *uf,
                   const double *uo, const double *ug, const double *h0,
                   const double *c0, const double *h, const double *c,
                   const double *gh, const double *gc,
                   double *dpi, double *dpf, double *dpo, double *dpg,
                   double *dui, double *duf, double *duo, double *dug,
                   double *dh0, double *dc0)
{
    double *acc = (double *)calloc((size_t)B * (size_t)H * 4, sizeof(double));
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t j = 0; j < H; ++j) {
            double lc = 0.0, lh = 0.0;
            double su[4] = {0, 0, 0, 0};
            for (int64_t t = L - 1; t >= 0; --t) {
                size_t kk = IDX(bb, t, j);
                lh += gh[kk];
                if (gc) lc += gc[kk];
                double hp = t == 0 ? (h0 ? h0[bb * H + j] : 0.0) : h[IDX(bb, t - 1, j)];
                double cp = t == 0 ? (c0 ? c0[bb * H + j] : 0.0) : c[IDX(bb, t - 1, j)];
                double cn, hn, J[4], dcdp[4], dhdp[4];
                orc_lstm_cell(cp, hp, pi[kk], pf[kk], po[kk], pg[kk], ui[j],
                              uf[j], uo[j], ug[j], &cn, &hn, J, dcdp, dhdp);
                double d[4];
                for (int q = 0; q < 4; ++q) d[q] = dcdp[q] * lc + dhdp[q] * lh;
                dpi[kk] = d[0];
                dpf[kk] = d[1];
                dpo[kk] = d[2];
                dpg[kk] = d[3];
                for (int q = 0; q < 4; ++q) su[q] += d[q] * hp;
                /* lambda_{t-1} = J^T lambda_t  (rows c,h; columns c',h') */
                double nlc = J[0] * lc + J[2] * lh;
                double nlh = J[1] * lc + J[3] * lh;
                lc = nlc;
                lh = nlh;
            }
            if (dh0) dh0[bb * H + j] = lh;
            if (dc0) dc0[bb * H + j] = lc;
            for (int q = 0; q < 4; ++q) acc[(bb * H + j) * 4 + q] = su[q];
        }
    double *outs[4] = {dui, duf, duo, dug};
    for (int q = 0; q < 4; ++q) {
        if (!outs[q]) continue;
        for (int64_t j = 0; j < H; ++j) {
            double a = 0;
            for (int64_t bb = 0; bb < B; ++bb) a += acc[(bb * H + j) * 4 + q];
            outs[q][j] = a;
        }
    }
    free(acc);
}

/* -------------------------------------------------------------------------
 * GRU cell with dense recurrence inside heads of k channels (k <= 8): the
 * diagonal GRU cell above with its weight vectors u replaced by one k x k
 * matrix per head (DEER summary page, limitations paragraph: dense
 * Jacobians; its GRU with heads of 8 channels).  Reading: each U acts on the
 * state vector where the diagonal cell multiplies elementwise by u, so a
 * diagonal U is exactly the diagonal cell:
 *   z = sig(pz + Uz h), r = sig(pr + Ur h), c = tanh(pc + Uc (r*h)),
 *   f = (1 - z)*h + z*c         (vectors of k, '*' elementwise)
 * U is row-major: U[i*k + l] takes component l of its operand into i.
 * Outputs f[k]; optionally J[k*k] = df/dh (row i, column l: d f_i / d h_l)
 * and the gates z, r, c, s = r*h (4 x k) for the backward pass.
 * ------------------------------------------------------------------------- */
void orc_hgru_cell(int k, const double *h, const double *pz, const double *pr,
                   const double *pc, const double *Uz, const double *Ur,
                   const double *Uc, double *f, double *J, double *gates)
{
    double z[8], r[8], s[8], c[8];
    for (int i = 0; i < k; ++i) {
        double az = pz[i], ar = pr[i];
        for (int l = 0; l < k; ++l) {
            az += Uz[i * k + l] * h[l];
            ar += Ur[i * k + l] * h[l];
        }
        z[i] = sigm(az);
        r[i] = sigm(ar);
        s[i] = r[i] * h[i];
    }
    for (int i = 0; i < k; ++i) {
        double ac = pc[i];
        for (int m = 0; m < k; ++m) ac += Uc[i * k + m] * s[m];
        c[i] = tanh(ac);
        f[i] = (1.0 - z[i]) * h[i] + z[i] * c[i];
    }
    if (J) {
        /* ds_m/dh_l = [m == l] r_m + h_m r_m (1 - r_m) Ur[m][l]
           dc_i/dh_l = (1 - c_i^2) sum_m Uc[i][m] ds_m/dh_l
           df_i/dh_l = [i == l](1 - z_i) + (c_i - h_i) z_i (1 - z_i) Uz[i][l]
                       + z_i dc_i/dh_l */
        for (int i = 0; i < k; ++i)
            for (int l = 0; l < k; ++l) {
                double dc = 0.0;
                for (int m = 0; m < k; ++m) {
                    double ds = (m == l ? r[m] : 0.0) + h[m] * r[m] * (1.0 - r[m]) * Ur[m * k + l];
                    dc += Uc[i * k + m] * ds;
                }
                dc *= 1.0 - c[i] * c[i];
                J[i * k + l] = (i == l ? 1.0 - z[i] : 0.0)
                               + (c[i] - h[i]) * z[i] * (1.0 - z[i]) * Uz[i * k + l]
                               + z[i] * dc;
            }
    }
    if (gates)
        for (int i = 0; i < k; ++i) {
            gates[i] = z[i];
            gates[k + i] = r[i];
            gates[2 * k + i] = c[i];
            gates[3 * k + i] = s[i];
        }
}

/* Index of component i of head n at (b, t) in a [B, L, NH, k] tensor. */
#define HIDX(b, t, n, i) ((((size_t)(b) * (size_t)L + (size_t)(t)) * (size_t)NH + (size_t)(n)) * (size_t)k + (size_t)(i))

/* Sequential rollout of the head GRU: tensors [B, L, NH, k], U [NH, k, k],
   h0 [B, NH, k] or NULL. */
void orc_hgru_rollout(int64_t B, int64_t L, int64_t NH, int k,
                      const double *pz, const double *pr, const double *pc,
                      const double *Uz, const double *Ur, const double *Uc,
                      const double *h0, double *h)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t n = 0; n < NH; ++n) {
            double x[8], f[8];
            for (int i = 0; i < k; ++i) x[i] = h0 ? h0[((size_t)bb * NH + n) * k + i] : 0.0;
            const size_t u = (size_t)n * k * k;
            for (int64_t t = 0; t < L; ++t) {
                size_t e = HIDX(bb, t, n, 0);
                orc_hgru_cell(k, x, pz + e, pr + e, pc + e, Uz + u, Ur + u, Uc + u, f, NULL, NULL);
                for (int i = 0; i < k; ++i) {
                    x[i] = f[i];
                    h[e + i] = f[i];
                }
            }
        }
}

/* Newton's method for the head GRU from s = 0 (or s_init), as orc_gru_newton: the
   linearised system is block bi-diagonal with the k x k Jacobians of the
   cell, solved by forward substitution delta_t = J_t delta_{t-1} - r_t. */
int orc_hgru_newton(int64_t B, int64_t L, int64_t NH, int k,
                    const double *pz, const double *pr, const double *pc,
                    const double *Uz, const double *Ur, const double *Uc,
                    const double *h0, const double *s_init, double tol, int cap,
                    double *s, int *converged, double *trace)
{
    size_t N = (size_t)B * (size_t)L * (size_t)NH * (size_t)k;
    double *F = (double *)malloc(N * sizeof(double));
    double *Jm = (double *)malloc(N * (size_t)k * sizeof(double));
    if (s_init)
        memcpy(s, s_init, N * sizeof(double));
    else
        memset(s, 0, N * sizeof(double));
    *converged = 0;
    int it;
    for (it = 1; it <= cap; ++it) {
        double e = 0.0;
#pragma omp parallel for collapse(2) schedule(static) reduction(max : e)
        for (int64_t bb = 0; bb < B; ++bb)
            for (int64_t n = 0; n < NH; ++n) {
                const size_t u = (size_t)n * k * k;
                double prev[8];
                for (int64_t t = 0; t < L; ++t) {
                    size_t ee = HIDX(bb, t, n, 0);
                    for (int i = 0; i < k; ++i)
                        prev[i] = t > 0 ? s[HIDX(bb, t - 1, n, i)]
                                        : (h0 ? h0[((size_t)bb * NH + n) * k + i] : 0.0);
                    orc_hgru_cell(k, prev, pz + ee, pr + ee, pc + ee, Uz + u, Ur + u, Uc + u,
                                  F + ee, Jm + ee * k, NULL);
                }
                double d[8] = {0}, dn[8], em = 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    size_t ee = HIDX(bb, t, n, 0);
                    for (int i = 0; i < k; ++i) {
                        double v = F[ee + i] - s[ee + i];
                        for (int l = 0; l < k; ++l) v += Jm[(ee + i) * k + l] * d[l];
                        dn[i] = v;
                    }
                    for (int i = 0; i < k; ++i) {
                        d[i] = dn[i];
                        em = absmax_update(em, d[i]);
                        s[ee + i] += d[i];
                    }
                }
                if (em > e) e = em;
            }
        if (trace) trace[it - 1] = e;
        if (e <= tol) {
            *converged = 1;
            break;
        }
    }
    free(F);
    free(Jm);
    return it > cap ? cap : it;
}

/* Backpropagation through time for L = sum_t g_t . h_t through the head GRU,
   given the forward states h:
     lambda_t = g_t + J_{t+1}^T lambda_{t+1}
     dL/dpz_i = lambda_i (c_i - h_i) z_i (1 - z_i)
     dL/dpc_i = lambda_i z_i (1 - c_i^2)
     dL/dpr_m = h_m r_m (1 - r_m) sum_i Uc[i][m] dL/dpc_i
     dL/dUz[i][l] += dL/dpz_i h_l,  dL/dUr[m][l] += dL/dpr_m h_l,
     dL/dUc[i][m] += dL/dpc_i s_m   (h the state entering the step)
     dL/dh0 = J_0^T lambda_0.
   dU [NH, k, k] is summed over b and t and written; dh0 may be NULL. */
void orc_hgru_bptt(int64_t B, int64_t L, int64_t NH, int k,
                   const double *pz, const double *pr, const double *pc,
                   const double *Uz, const double *Ur, const double *Uc,
                   const double *h0, const double *h, const double *g,
                   double *dpz, double *dpr, double *dpc,
                   double *dUz, double *dUr, double *dUc, double *dh0)
{
    const size_t kk = (size_t)k * k;
    double *acc = (double *)calloc((size_t)B * NH * 3 * kk, sizeof(double));
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bb = 0; bb < B; ++bb)
        for (int64_t n = 0; n < NH; ++n) {
            const size_t u = (size_t)n * kk;
            double *az = acc + ((size_t)bb * NH + n) * 3 * kk, *ar = az + kk, *ac = ar + kk;
            double lam[8] = {0}, prev[8], f[8], J[64], gt[32];
            for (int64_t t = L - 1; t >= 0; --t) {
                size_t ee = HIDX(bb, t, n, 0);
                for (int i = 0; i < k; ++i) {
                    lam[i] += g[ee + i];
                    prev[i] = t > 0 ? h[HIDX(bb, t - 1, n, i)]
                                    : (h0 ? h0[((size_t)bb * NH + n) * k + i] : 0.0);
                }
                orc_hgru_cell(k, prev, pz + ee, pr + ee, pc + ee, Uz + u, Ur + u, Uc + u, f, J, gt);
                const double *z = gt, *r = gt + k, *c = gt + 2 * k, *sv = gt + 3 * k;
                for (int i = 0; i < k; ++i) {
                    dpz[ee + i] = lam[i] * (c[i] - prev[i]) * z[i] * (1.0 - z[i]);
                    dpc[ee + i] = lam[i] * z[i] * (1.0 - c[i] * c[i]);
                }
                for (int m = 0; m < k; ++m) {
                    double v = 0.0;
                    for (int i = 0; i < k; ++i) v += Uc[u + i * k + m] * dpc[ee + i];
                    dpr[ee + m] = prev[m] * r[m] * (1.0 - r[m]) * v;
                }
                for (int i = 0; i < k; ++i)
                    for (int l = 0; l < k; ++l) {
                        az[i * k + l] += dpz[ee + i] * prev[l];
                        ar[i * k + l] += dpr[ee + i] * prev[l];
                        ac[i * k + l] += dpc[ee + i] * sv[l];
                    }
                double nl[8];
                for (int l = 0; l < k; ++l) {
                    double v = 0.0;
                    for (int i = 0; i < k; ++i) v += J[i * k + l] * lam[i];
                    nl[l] = v;
                }
                for (int l = 0; l < k; ++l) lam[l] = nl[l];
            }
            if (dh0)
                for (int i = 0; i < k; ++i) dh0[((size_t)bb * NH + n) * k + i] = lam[i];
        }
    for (int64_t n = 0; n < NH; ++n)
        for (size_t q = 0; q < kk; ++q) {
            double a0 = 0, a1 = 0, a2 = 0;
            for (int64_t bb = 0; bb < B; ++bb) {
                const double *a = acc + ((size_t)bb * NH + n) * 3 * kk;
                a0 += a[q];
                a1 += a[kk + q];
                a2 += a[2 * kk + q];
            }
            dUz[n * kk + q] = a0;
            dUr[n * kk + q] = a1;
            dUc[n * kk + q] = a2;
        }
    free(acc);
}

/* Number of OpenMP threads the parallel loops above use (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}
