// cells.hpp -- fp32 device evaluation of the two diagonal-recurrence cells,
// their Jacobians with respect to the previous state, and their partials
// with respect to the gate pre-activations.
//
// GRU-style cell (ParaGRU; ParaRNN page, Fig. 2 caption: diagonal
// Jacobian).  Per channel, with h the previous state:
//   z = s(pz + uz h), r = s(pr + ur h), c = tanh(pc + uc r h),
//   F = h + z (c - h)
//   dF/dh = (1 - z) + z(1-z) uz (c - h) + z (1 - c^2) uc (r + h r(1-r) ur)
//
// LSTM-style cell (ParaLSTM; Fig. 2 caption: 2x2 block-diagonal Jacobian).
// State (c, h), previous (c', h'):
//   i, f, o = s(p + u h'), g = tanh(pg + ug h'), c = f c' + i g, h = o tanh(c)
//   kappa = dc/dh' = c' f(1-f) uf + g i(1-i) ui + i (1-g^2) ug
//   J = [[f, kappa], [o(1-tanh^2 c) f, o(1-o) uo tanh c + o(1-tanh^2 c) kappa]]
#pragma once

#include "common.hpp"

namespace prn {

__device__ __forceinline__ void gru_f_j(float h, float pz, float pr, float pc, float uz,
                                        float ur, float uc, float &F, float &J) {
    const float z = sigmoid(fmaf(uz, h, pz));
    const float r = sigmoid(fmaf(ur, h, pr));
    const float c = tanh_fast(fmaf(uc, r * h, pc));
    const float cmh = c - h;
    F = fmaf(z, cmh, h);
    const float omz = 1.0f - z;
    const float omc2 = fmaf(-c, c, 1.0f);
    const float drh = fmaf(h * (r - r * r), ur, r);  // d(r h)/dh
    J = fmaf(z * omc2 * uc, drh, fmaf(z * omz * uz, cmh, omz));
}

// Jacobian and the partials dF/dpz, dF/dpr, dF/dpc at previous state h; also r.
__device__ __forceinline__ void gru_j_dp(float h, float pz, float pr, float pc, float uz,
                                         float ur, float uc, float &J, float &dz, float &dr,
                                         float &dc, float &r_out) {
    const float z = sigmoid(fmaf(uz, h, pz));
    const float r = sigmoid(fmaf(ur, h, pr));
    const float c = tanh_fast(fmaf(uc, r * h, pc));
    const float cmh = c - h;
    const float omz = 1.0f - z;
    const float zomz = z * omz;
    const float omc2 = fmaf(-c, c, 1.0f);
    const float rr = r - r * r;
    const float drh = fmaf(h * rr, ur, r);
    dz = zomz * cmh;
    dc = z * omc2;
    dr = dc * uc * h * rr;
    J = fmaf(dc * uc, drh, fmaf(zomz * uz, cmh, omz));
    r_out = r;
}

// The GRU's Newton map at one position, on gate inputs and weights
// pre-scaled into the exp2 domain (xz, xr and wz, wr by -log2 e; xc and wc by
// -2 log2 e), so that each gate is one fma, exp2, add and reciprocal.  Gives
// J = dF/dh and beta = F - s at previous state hp.  Rewritten to save
// instructions, exactly equal in real arithmetic to gru_f_j above:
//   - with sc the sigmoid behind c = 2 sc - 1, 1 - c^2 = 4 sc (1 - sc), so
//     uc enters as uc4 = 4 uc;
//   - h r (1 - r) = rh - rh r with rh = r h, which the c gate needs anyway;
//   - (1 - z) + z inner = 1 + z (inner - 1), (1 - z) uz = uz - z uz, and
//     the -1 folds into the multiply-add of the c term.
struct GruScaledW {
    float wz, wr, wc;   // the gates' weights, scaled as their inputs
    float uz, ur, uc4;  // the Jacobian's: uz, ur as given, 4 uc
};
__device__ __forceinline__ GruScaledW gru_scaled_weights(float uz, float ur, float uc) {
    return {-kLog2e * uz, -kLog2e * ur, -2.0f * kLog2e * uc, uz, ur, 4.0f * uc};
}
__device__ __forceinline__ void gru_map_scaled(const GruScaledW &w, float hp, float xz, float xr, float xc,
                                               float s, float &J, float &beta) {
    const float z = fast_rcp(1.0f + fast_exp2(fmaf(w.wz, hp, xz)));
    const float r = fast_rcp(1.0f + fast_exp2(fmaf(w.wr, hp, xr)));
    const float rh = r * hp;
    const float sc = fast_rcp(1.0f + fast_exp2(fmaf(w.wc, rh, xc)));
    const float cmh = fmaf(2.0f, sc, -1.0f) - hp;  // c - h
    beta = fmaf(z, cmh, hp) - s;
    const float drh = fmaf(fmaf(-rh, r, rh), w.ur, r);            // d(r h)/dh
    const float v = fmaf(fmaf(-sc, sc, sc) * w.uc4, drh, -1.0f);  // (1 - c^2) uc d(r h)/dh - 1
    J = fmaf(z, fmaf(fmaf(-z, w.uz, w.uz), cmh, v), 1.0f);
}

// gru_map_scaled at hp = 0 and s = 0: Newton's first iteration from the
// zero iterate at every position whose previous state is that iterate's.
// The terms that vanish are dropped, so it gives the same bits as
// gru_map_scaled there (fma(w, 0, x) = x, fma(-0 r, ., r) = r, ...).
__device__ __forceinline__ void gru_map_scaled0(const GruScaledW &w, float xz, float xr, float xc, float &J,
                                                float &beta) {
    const float z = fast_rcp(1.0f + fast_exp2(xz));
    const float r = fast_rcp(1.0f + fast_exp2(xr));
    const float sc = fast_rcp(1.0f + fast_exp2(xc));
    const float c = fmaf(2.0f, sc, -1.0f);
    beta = z * c;
    const float v = fmaf(fmaf(-sc, sc, sc) * w.uc4, r, -1.0f);
    J = fmaf(z, fmaf(fmaf(-z, w.uz, w.uz), c, v), 1.0f);
}

struct Lstm2 {
    float Fc, Fh;
    float j00, j01, j10, j11;
};

__device__ __forceinline__ Lstm2 lstm_f_j(float cp, float hp, float pi, float pf, float po,
                                          float pg, float ui, float uf, float uo, float ug) {
    const float i = sigmoid(fmaf(ui, hp, pi));
    const float f = sigmoid(fmaf(uf, hp, pf));
    const float o = sigmoid(fmaf(uo, hp, po));
    const float g = tanh_fast(fmaf(ug, hp, pg));
    const float c = fmaf(f, cp, i * g);
    const float tc = tanh_fast(c);
    const float dtc = fmaf(-tc, tc, 1.0f);
    const float kappa = fmaf(cp * (f - f * f), uf, fmaf(g * (i - i * i), ui, i * fmaf(-g, g, 1.0f) * ug));
    const float odtc = o * dtc;
    Lstm2 r;
    r.Fc = c;
    r.Fh = o * tc;
    r.j00 = f;
    r.j01 = kappa;
    r.j10 = odtc * f;
    r.j11 = fmaf((o - o * o) * uo, tc, odtc * kappa);
    return r;
}

// LSTM partials for the adjoint: Jacobian plus dc/dp (i, f, g; dc/dpo = 0)
// and dh/dp (i, f, o, g).
struct LstmAdj {
    float j00, j01, j10, j11;
    float dci, dcf, dcg;
    float dhi, dhf, dho, dhg;
    float odtc;  // o (1 - tanh^2 c): dh/dp_{i,f,g} = odtc dc/dp_{i,f,g}, j10 = odtc j00
};

__device__ __forceinline__ LstmAdj lstm_adj(float cp, float hp, float pi, float pf, float po,
                                            float pg, float ui, float uf, float uo, float ug) {
    const float i = sigmoid(fmaf(ui, hp, pi));
    const float f = sigmoid(fmaf(uf, hp, pf));
    const float o = sigmoid(fmaf(uo, hp, po));
    const float g = tanh_fast(fmaf(ug, hp, pg));
    const float c = fmaf(f, cp, i * g);
    const float tc = tanh_fast(c);
    const float dtc = fmaf(-tc, tc, 1.0f);
    const float odtc = o * dtc;
    LstmAdj a;
    a.dci = g * (i - i * i);
    a.dcf = cp * (f - f * f);
    a.dcg = i * fmaf(-g, g, 1.0f);
    const float kappa = fmaf(a.dcf, uf, fmaf(a.dci, ui, a.dcg * ug));
    a.j00 = f;
    a.j01 = kappa;
    a.j10 = odtc * f;
    a.j11 = fmaf((o - o * o) * uo, tc, odtc * kappa);
    a.dhi = odtc * a.dci;
    a.dhf = odtc * a.dcf;
    a.dho = (o - o * o) * tc;
    a.dhg = odtc * a.dcg;
    a.odtc = odtc;
    return a;
}

}  // namespace prn
