/*
 * Plain fp64 CPU oracle for the dense gated delta rule: Gated DeltaNet (scalar
 * decay) and Kimi Delta Attention (per-key-channel decay).  DeltaNet is the
 * case alpha = 1.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this code; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source with the HIP library.
 *
 * Sources (reading slides "Linear Attention Architectures: Mechanisms,
 * Trade-offs, and Cross-Layer Routing"):
 *   - slide "The memory maps key features into value space" (Eqs. 4-10):
 *     W in R^{dv x dk}; read y = W phi(q) on the state AFTER the write.
 *   - slide "DeltaNet writes a correction to the current association"
 *     (Eq. 14): r = v - W_old kappa; W_new = W_old + beta r kappa^T.
 *   - slide "GDN and KDA change the granularity of forgetting" (Eqs. 15-20):
 *     GDN  r = v - alpha W_old kappa;  W_new = alpha W_old + beta r kappa^T
 *     KDA  r = v - W_old D kappa;      W_new = W_old D + beta r kappa^T,
 *     D = Diag(alpha) on the right, i.e. on the key channels.
 *
 * The state is stored transposed, S = W^T with shape [dk, dv] (row = key
 * channel), so KDA's right-multiplication by D scales the rows of S.
 * Readings: phi is the identity (keys arrive already normalised by the
 * caller); no 1/sqrt(d) query scale; the decay-adjusted residual of
 * Eqs. 15-17 is used.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 *   q, k : [B,T,H,dk]    v : [B,T,H,dv]
 *   alpha: [B,T,H] (kda == 0) or [B,T,H,dk] (kda == 1)
 *   beta : [B,T,H]
 *   S0   : [B,H,dk,dv] initial state, or NULL for zeros
 *   S    : [B,H,dk,dv] final state (out)
 *   o    : [B,T,H,dv]  outputs o_t = S_t^T q_t
 */
int orc_gdn(int B, int T, int H, int dk, int dv, int kda, const float* q, const float* k,
            const float* v, const float* alpha, const float* beta, const double* S0, double* S,
            double* o) {
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || (kda != 0 && kda != 1)) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            size_t sb = ((size_t)b * H + h) * (size_t)dk * dv;
            double* st = S + sb;
            if (S0)
                memcpy(st, S0 + sb, sizeof(double) * (size_t)dk * dv);
            else
                memset(st, 0, sizeof(double) * (size_t)dk * dv);
            double* pred = (double*)malloc(sizeof(double) * dv);
            for (int t = 0; t < T; ++t) {
                size_t bth = ((size_t)b * T + t) * H + h;
                const float* qt = q + bth * dk;
                const float* kt = k + bth * dk;
                const float* vt = v + bth * dv;
                double be = beta[bth];
                /* decay: S~ = alpha S (GDN) or Diag(alpha) S (KDA) */
                for (int i = 0; i < dk; ++i) {
                    double a = kda ? (double)alpha[bth * dk + i] : (double)alpha[bth];
                    for (int c = 0; c < dv; ++c) st[(size_t)i * dv + c] *= a;
                }
                /* prediction at the current key from the decayed state: S~^T k */
                for (int c = 0; c < dv; ++c) pred[c] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int c = 0; c < dv; ++c) pred[c] += (double)kt[i] * st[(size_t)i * dv + c];
                /* delta write: S = S~ + beta k (v - pred)^T */
                for (int i = 0; i < dk; ++i)
                    for (int c = 0; c < dv; ++c)
                        st[(size_t)i * dv + c] += be * (double)kt[i] * ((double)vt[c] - pred[c]);
                /* read after the write: o = S^T q */
                double* ot = o + bth * dv;
                for (int c = 0; c < dv; ++c) ot[c] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int c = 0; c < dv; ++c) ot[c] += (double)qt[i] * st[(size_t)i * dv + c];
            }
            free(pred);
        }
    return 0;
}

/*
 * GDN2 (slide "GDN2 separates key-side erase and value-side write",
 * Eqs. 21-24): with the KDA decay on the key channels,
 *   W~ = W_old D_alpha,  e = b (.) kappa,  z = w (.) v,
 *   W_new = W~ + (z - W~ e) kappa^T,
 * b in (0,1)^{dk} steering what is erased and w in (0,1)^{dv} what is
 * written; the outer product keeps kappa.  b = w = beta 1 is KDA.  In the
 * transposed state S = W^T: S~ = Diag(alpha) S, r = z - S~^T e,
 * S = S~ + kappa r^T, and the read o = S^T q after the write.
 *   q, k, alpha, bvec : [B,T,H,dk]    v, wvec : [B,T,H,dv]
 */
int orc_gdn2(int B, int T, int H, int dk, int dv, const float* q, const float* k, const float* v,
             const float* alpha, const float* bvec, const float* wvec, const double* S0, double* S,
             double* o) {
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            size_t sb = ((size_t)b * H + h) * (size_t)dk * dv;
            double* st = S + sb;
            if (S0)
                memcpy(st, S0 + sb, sizeof(double) * (size_t)dk * dv);
            else
                memset(st, 0, sizeof(double) * (size_t)dk * dv);
            double* r = (double*)malloc(sizeof(double) * dv);
            for (int t = 0; t < T; ++t) {
                size_t bth = ((size_t)b * T + t) * H + h;
                const float* qt = q + bth * dk;
                const float* kt = k + bth * dk;
                const float* vt = v + bth * dv;
                const float* at = alpha + bth * dk;
                const float* bt = bvec + bth * dk;
                const float* wt = wvec + bth * dv;
                for (int i = 0; i < dk; ++i)
                    for (int c = 0; c < dv; ++c) st[(size_t)i * dv + c] *= (double)at[i];
                /* r = z - S~^T e with e = b (.) kappa, z = w (.) v */
                for (int c = 0; c < dv; ++c) r[c] = (double)wt[c] * (double)vt[c];
                for (int i = 0; i < dk; ++i) {
                    const double e = (double)bt[i] * (double)kt[i];
                    for (int c = 0; c < dv; ++c) r[c] -= e * st[(size_t)i * dv + c];
                }
                /* S = S~ + kappa r^T */
                for (int i = 0; i < dk; ++i)
                    for (int c = 0; c < dv; ++c) st[(size_t)i * dv + c] += (double)kt[i] * r[c];
                double* ot = o + bth * dv;
                for (int c = 0; c < dv; ++c) ot[c] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int c = 0; c < dv; ++c) ot[c] += (double)qt[i] * st[(size_t)i * dv + c];
            }
            free(r);
        }
    return 0;
}
