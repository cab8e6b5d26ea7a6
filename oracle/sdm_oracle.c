/*
 * Plain fp64 CPU oracle for Sparse Delta Memory (SDM): product-key addressing
 * and the sparse decay / delta-update / read recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this code; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source with the HIP library.
 *
 * Sources (reading slides "Sparse Delta Memory: Scaling the State of Linear
 * RNNs through Sparsity"):
 *   - slide "Product keys select addresses without scoring every slot":
 *     score of slot (a,b) is the outer SUM k'_1[a] + k'_2[b]; keep each half's
 *     top-k, form the k^2 candidate sums, select top-W (write) / top-R (read),
 *     softmax over the selected scores.
 *   - slide "Selected slots decay and update; other slots persist",
 *     Eqs. (3)-(5): decay only the selected write slots, delta update, slots
 *     outside the write set unchanged, read y_t from the UPDATED table.
 *   - slide "A v1 inconsistency matters for reproducing the update": the
 *     figure's shared prediction v_hat = sum_i k^(i) M~[i] (residual_mode 0)
 *     versus Eq. (4)'s per-slot residual v - M~[i] (residual_mode 1).
 *
 * Readings where the slides are silent (each one is listed in the design
 * notes):
 *   - slot numbering: slot(a,b) = a*sqrtN + b, a indexing half 1;
 *   - ranking: score descending, ties to the lowest index, at both stages;
 *     -0 and +0 compare equal (plain float comparison);
 *   - the selection key is the fp32 sum of the two fp32 half scores (the
 *     value a GPU ranks on); every other quantity is fp64;
 *   - returned indices are in rank order; weights are a plain softmax of the
 *     selected fp32 keys (no temperature);
 *   - alpha_t, beta_t are scalars per (batch, token, head).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    float key;   /* fp32 ranking value */
    int32_t id;  /* index used to break ties (lower wins) */
} ranked_t;

/* Rank order: larger key first; equal keys -> smaller id first.
 * -0.0f == +0.0f under C float comparison, so they tie. */
static int rank_cmp(const void* pa, const void* pb) {
    const ranked_t* a = (const ranked_t*)pa;
    const ranked_t* b = (const ranked_t*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    if (a->id < b->id) return -1;
    if (a->id > b->id) return 1;
    return 0;
}

/*
 * Product-key addressing for P independent problems.
 *   s1, s2 : [P, sqrtN] fp32 half scores
 *   k      : per-half top-k, 1 <= k <= sqrtN
 *   budget : number of selected slots (W or R), 1 <= budget <= k*k
 *   idx    : [P, budget] selected slots in rank order
 *   wt     : [P, budget] softmax weights (fp64)
 * Returns 0, or -1 on invalid arguments.
 */
int orc_sdm_address(int P, int sqrtN, const float* s1, const float* s2, int k, int budget,
                    int32_t* idx, double* wt) {
    if (P < 0 || sqrtN <= 0 || k <= 0 || k > sqrtN || budget <= 0 || budget > k * k) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int p = 0; p < P; ++p) {
        const float* h1 = s1 + (size_t)p * sqrtN;
        const float* h2 = s2 + (size_t)p * sqrtN;
        ranked_t* r1 = (ranked_t*)malloc(sizeof(ranked_t) * sqrtN);
        ranked_t* r2 = (ranked_t*)malloc(sizeof(ranked_t) * sqrtN);
        ranked_t* cand = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)k * k);
        /* step 1: each half's top-k */
        for (int a = 0; a < sqrtN; ++a) { r1[a].key = h1[a]; r1[a].id = a; }
        for (int b = 0; b < sqrtN; ++b) { r2[b].key = h2[b]; r2[b].id = b; }
        qsort(r1, sqrtN, sizeof(ranked_t), rank_cmp);
        qsort(r2, sqrtN, sizeof(ranked_t), rank_cmp);
        /* step 2: the k^2 candidate sums, slot = a*sqrtN + b */
        int n = 0;
        for (int i = 0; i < k; ++i)
            for (int j = 0; j < k; ++j) {
                int a = r1[i].id, b = r2[j].id;
                float s = h1[a] + h2[b]; /* one fp32 round-to-nearest-even add */
                cand[n].key = s;
                cand[n].id = a * sqrtN + b;
                ++n;
            }
        /* step 3: top-budget of the candidates */
        qsort(cand, n, sizeof(ranked_t), rank_cmp);
        /* step 4: softmax over the selected scores */
        double mx = (double)cand[0].key, z = 0.0;
        for (int m = 0; m < budget; ++m) z += exp((double)cand[m].key - mx);
        for (int m = 0; m < budget; ++m) {
            idx[(size_t)p * budget + m] = cand[m].id;
            wt[(size_t)p * budget + m] = exp((double)cand[m].key - mx) / z;
        }
        free(r1);
        free(r2);
        free(cand);
    }
    return 0;
}

/*
 * The SDM recurrence given the addressing, one token at a time.
 *   idx_w, wt_w : [B,T,H,W]  write slots (distinct within a token) and weights
 *   idx_r, wt_r : [B,T,H,R]  read slots and weights
 *   v           : [B,T,H,dv] values
 *   alpha, beta : [B,T,H]    forget gate and input gate
 *   M           : [B,H,N,dv] table, updated in place
 *   y           : [B,T,H,dv] reads
 *   residual_mode 0 (shared prediction, figure form):
 *       M~[i] = alpha*M[i];  v_hat = sum_n wt_n M~[i_n];
 *       M[i_n] = M~[i_n] + beta*wt_n*(v - v_hat)
 *   residual_mode 1 (per-slot, Eq. (4) as printed):
 *       M[i_n] = M~[i_n] + beta*wt_n*(v - M~[i_n])
 *   then y = sum_m wt_r_m M[j_m] on the updated table.
 * Slots not in the token's write set are never touched.
 * Given the addressing every operation above acts on one column c of d_v at a
 * time (the shared prediction v_hat[c] included), so the columns are separate
 * recurrences; the loops run over (b, h, block of ORC_COLS columns) in
 * parallel, the token loop inside in the plain sequential order.  Each
 * column's arithmetic is the same sequence of fp64 operations whatever the
 * block size.
 */
#define ORC_COLS 64
int orc_sdm_recurrence(int B, int T, int H, long long N, int dv, int W, int R, int residual_mode,
                       const int32_t* idx_w, const double* wt_w, const int32_t* idx_r,
                       const double* wt_r, const float* v, const float* alpha, const float* beta,
                       double* M, double* y) {
    if (B < 0 || T < 0 || H <= 0 || N <= 0 || dv <= 0 || W <= 0 || R <= 0) return -1;
    if (residual_mode != 0 && residual_mode != 1) return -1;
    const int nblk = (dv + ORC_COLS - 1) / ORC_COLS;
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int blk = 0; blk < nblk; ++blk) {
                const int c0 = blk * ORC_COLS;
                const int c1 = c0 + ORC_COLS < dv ? c0 + ORC_COLS : dv;
                double* tab = M + ((size_t)b * H + h) * (size_t)N * dv;
                double* mt = (double*)malloc(sizeof(double) * (size_t)W * dv); /* M~ rows */
                double* vhat = (double*)malloc(sizeof(double) * dv);
                for (int t = 0; t < T; ++t) {
                    size_t bth = ((size_t)b * T + t) * H + h;
                    const int32_t* iw = idx_w + bth * W;
                    const double* gw = wt_w + bth * W;
                    const int32_t* ir = idx_r + bth * R;
                    const double* gr = wt_r + bth * R;
                    const float* vt = v + bth * dv;
                    double a = alpha[bth], be = beta[bth];
                    /* Eq. (3): decay of the selected write slots */
                    for (int n = 0; n < W; ++n)
                        for (int c = c0; c < c1; ++c)
                            mt[(size_t)n * dv + c] = a * tab[(size_t)iw[n] * dv + c];
                    if (residual_mode == 0) {
                        for (int c = c0; c < c1; ++c) {
                            double s = 0.0;
                            for (int n = 0; n < W; ++n) s += gw[n] * mt[(size_t)n * dv + c];
                            vhat[c] = s;
                        }
                        for (int n = 0; n < W; ++n)
                            for (int c = c0; c < c1; ++c)
                                tab[(size_t)iw[n] * dv + c] =
                                    mt[(size_t)n * dv + c] + be * gw[n] * ((double)vt[c] - vhat[c]);
                    } else {
                        for (int n = 0; n < W; ++n)
                            for (int c = c0; c < c1; ++c)
                                tab[(size_t)iw[n] * dv + c] =
                                    mt[(size_t)n * dv + c] +
                                    be * gw[n] * ((double)vt[c] - mt[(size_t)n * dv + c]);
                    }
                    /* Eq. (5): read after writing */
                    double* yt = y + bth * dv;
                    for (int c = c0; c < c1; ++c) {
                        double s = 0.0;
                        for (int m = 0; m < R; ++m) s += gr[m] * tab[(size_t)ir[m] * dv + c];
                        yt[c] = s;
                    }
                }
                free(mt);
                free(vhat);
            }
    return 0;
}

/*
 * Gradient of the recurrence above (its vector-Jacobian product), computed the
 * way the Sparse Delta Memory slides' backup "Backup: undoing writes avoids
 * repeated full-table snapshots" describes: the forward keeps, per token, the
 * rows its write set held before the token (T * W * dv values per (b, h)
 * instead of one table per chunk); the backward walks the tokens in reverse
 * with the table at M_t, and steps it back to M_{t-1} by restoring those rows.
 *
 *   idx_w .. beta : as orc_sdm_recurrence (the forward is re-run here)
 *   M0            : [B,H,N,dv] initial table (read only)
 *   dy            : [B,T,H,dv] gradient of the reads
 *   dM            : [B,H,N,dv] in: gradient of the final table M_T;
 *                               out: gradient of the initial table M_0
 *   dv_out        : [B,T,H,dv]  gradient of v
 *   dalpha, dbeta : [B,T,H]     gradients of the gates
 *   dwt_w, dwt_r  : [B,T,H,W], [B,T,H,R] gradients of the addressing weights
 *
 * Per token t in reverse (G = gradient of M_t, one row per slot):
 *   read    y = sum_m wr_m M_t[j_m]:   dwr_m = <M_t[j_m], dy_t>;  G[j_m] += wr_m dy_t
 *   write   with P_n = M_{t-1}[i_n] (restored), Mt_n = alpha P_n, G_n = G[i_n]:
 *     SHARED   r = v - sum_n w_n Mt_n,  M_t[i_n] = Mt_n + beta w_n r:
 *              dr = sum_n beta w_n G_n;  dv = dr;  dbeta = sum_n w_n <G_n, r>;
 *              dw_n = beta <G_n, r> - <Mt_n, dr>;  dMt_n = G_n - w_n dr
 *     PER_SLOT M_t[i_n] = Mt_n + beta w_n (v - Mt_n):
 *              dv = sum_n beta w_n G_n;  dbeta = sum_n w_n <G_n, v - Mt_n>;
 *              dw_n = beta <G_n, v - Mt_n>;  dMt_n = (1 - beta w_n) G_n
 *     dalpha = sum_n <P_n, dMt_n>;  G[i_n] = alpha dMt_n;  table row i_n = P_n.
 * Rows outside the token's write set pass G through unchanged.
 */
int orc_sdm_recurrence_backward(int B, int T, int H, long long N, int dv, int W, int R,
                                int residual_mode, const int32_t* idx_w, const double* wt_w,
                                const int32_t* idx_r, const double* wt_r, const float* v,
                                const float* alpha, const float* beta, const double* M0,
                                const double* dy, double* dM, double* dv_out, double* dalpha,
                                double* dbeta, double* dwt_w, double* dwt_r) {
    if (B < 0 || T < 0 || H <= 0 || N <= 0 || dv <= 0 || W <= 0 || R <= 0) return -1;
    if (residual_mode != 0 && residual_mode != 1) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const size_t tsz = (size_t)N * dv;
            double* tab = (double*)malloc(sizeof(double) * tsz);
            double* G = dM + ((size_t)b * H + h) * tsz;
            double* saved = (double*)malloc(sizeof(double) * ((size_t)T * W * dv + 1));
            double* mt = (double*)malloc(sizeof(double) * (size_t)W * dv);
            double* r = (double*)malloc(sizeof(double) * dv);
            double* dr = (double*)malloc(sizeof(double) * dv);
            memcpy(tab, M0 + ((size_t)b * H + h) * tsz, sizeof(double) * tsz);
            /* forward, keeping each token's pre-write rows */
            for (int t = 0; t < T; ++t) {
                size_t bth = ((size_t)b * T + t) * H + h;
                const int32_t* iw = idx_w + bth * W;
                const double* gw = wt_w + bth * W;
                const float* vt = v + bth * dv;
                double a = alpha[bth], be = beta[bth];
                double* sv = saved + (size_t)t * W * dv;
                for (int n = 0; n < W; ++n)
                    for (int c = 0; c < dv; ++c) {
                        sv[(size_t)n * dv + c] = tab[(size_t)iw[n] * dv + c];
                        mt[(size_t)n * dv + c] = a * sv[(size_t)n * dv + c];
                    }
                for (int c = 0; c < dv; ++c) {
                    double s = 0.0;
                    for (int n = 0; n < W; ++n) s += gw[n] * mt[(size_t)n * dv + c];
                    r[c] = (double)vt[c] - s;
                }
                for (int n = 0; n < W; ++n)
                    for (int c = 0; c < dv; ++c) {
                        double res = residual_mode == 0 ? r[c] : (double)vt[c] - mt[(size_t)n * dv + c];
                        tab[(size_t)iw[n] * dv + c] = mt[(size_t)n * dv + c] + be * gw[n] * res;
                    }
            }
            /* reverse sweep; tab holds M_t on entry to step t */
            for (int t = T - 1; t >= 0; --t) {
                size_t bth = ((size_t)b * T + t) * H + h;
                const int32_t* iw = idx_w + bth * W;
                const double* gw = wt_w + bth * W;
                const int32_t* ir = idx_r + bth * R;
                const double* gr = wt_r + bth * R;
                const float* vt = v + bth * dv;
                const double* dyt = dy + bth * dv;
                double a = alpha[bth], be = beta[bth];
                const double* sv = saved + (size_t)t * W * dv;
                /* read after writing */
                for (int m = 0; m < R; ++m) {
                    double s = 0.0;
                    for (int c = 0; c < dv; ++c) s += tab[(size_t)ir[m] * dv + c] * dyt[c];
                    dwt_r[bth * R + m] = s;
                    for (int c = 0; c < dv; ++c) G[(size_t)ir[m] * dv + c] += gr[m] * dyt[c];
                }
                /* the write, from the restored rows */
                for (int n = 0; n < W; ++n)
                    for (int c = 0; c < dv; ++c) mt[(size_t)n * dv + c] = a * sv[(size_t)n * dv + c];
                for (int c = 0; c < dv; ++c) {
                    double s = 0.0, g = 0.0;
                    for (int n = 0; n < W; ++n) {
                        s += gw[n] * mt[(size_t)n * dv + c];
                        g += be * gw[n] * G[(size_t)iw[n] * dv + c];
                    }
                    r[c] = (double)vt[c] - s;
                    dr[c] = g;
                    dv_out[bth * dv + c] = g;
                }
                double db = 0.0, da = 0.0;
                for (int n = 0; n < W; ++n) {
                    double* gn = G + (size_t)iw[n] * dv;
                    const double* mn = mt + (size_t)n * dv;
                    double gres = 0.0, mdr = 0.0;
                    for (int c = 0; c < dv; ++c) {
                        double res = residual_mode == 0 ? r[c] : (double)vt[c] - mn[c];
                        gres += gn[c] * res;
                        mdr += mn[c] * dr[c];
                    }
                    db += gw[n] * gres;
                    dwt_w[bth * W + n] = residual_mode == 0 ? be * gres - mdr : be * gres;
                    for (int c = 0; c < dv; ++c) {
                        double dmt = residual_mode == 0 ? gn[c] - gw[n] * dr[c]
                                                        : (1.0 - be * gw[n]) * gn[c];
                        da += sv[(size_t)n * dv + c] * dmt;
                        gn[c] = a * dmt;
                        tab[(size_t)iw[n] * dv + c] = sv[(size_t)n * dv + c];
                    }
                }
                dalpha[bth] = da;
                dbeta[bth] = db;
            }
            free(tab);
            free(saved);
            free(mt);
            free(r);
            free(dr);
        }
    return 0;
}

/*
 * Gradient of the addressing weights with respect to the score halves
 * (slide "Product keys select addresses without scoring every slot"): the
 * weights are a softmax of the selected scores s1[a] + s2[b], so with the
 * selection held fixed
 *   ds_m = wt_m (dwt_m - sum_j wt_j dwt_j),  ds1[a_m] += ds_m,  ds2[b_m] += ds_m,
 * where slot idx_m = a_m * sqrtN + b_m.  Halves outside every selected pair
 * get 0.
 *   idx, wt, dwt : [P, budget];  ds1, ds2 : [P, sqrtN] out.
 */
int orc_sdm_address_backward(int P, int sqrtN, int budget, const int32_t* idx, const double* wt,
                             const double* dwt, double* ds1, double* ds2) {
    if (P < 0 || sqrtN <= 0 || budget <= 0) return -1;
    for (int p = 0; p < P; ++p) {
        const int32_t* ip = idx + (size_t)p * budget;
        const double* w = wt + (size_t)p * budget;
        const double* dw = dwt + (size_t)p * budget;
        double* d1 = ds1 + (size_t)p * sqrtN;
        double* d2 = ds2 + (size_t)p * sqrtN;
        for (int a = 0; a < sqrtN; ++a) d1[a] = d2[a] = 0.0;
        double dot = 0.0;
        for (int m = 0; m < budget; ++m) dot += w[m] * dw[m];
        for (int m = 0; m < budget; ++m) {
            double ds = w[m] * (dw[m] - dot);
            d1[ip[m] / sqrtN] += ds;
            d2[ip[m] % sqrtN] += ds;
        }
    }
    return 0;
}

/*
 * The layer output after the read (Sparse Delta Memory slides, "Selected slots
 * decay and update; other slots persist": the read is followed by RMS-Norm,
 * output gating and head mixing).  The slides name the steps only; the plain
 * reading taken here, per (token, head) row of d values:
 *   o = y / sqrt(mean(y^2) + eps) * gamma * act(g)
 * with gamma [d] a per-channel weight shared by the heads, g the gate
 * pre-activation of the row, and act = SiLU (act 1, g * sigmoid(g)), the
 * logistic sigmoid (act 2) or none (act 0, the factor is 1).  Head mixing is
 * the dense output projection after this step and is not part of it.
 *   y, g : [P, d];  gamma : [d];  o : [P, d] out.
 * PARITY UNPINNED for the gate's activation choice (no printed value fixes
 * it); the RMS normalisation itself is the textbook definition.
 */
int orc_norm_gate(int P, int d, const float* y, const float* g, const float* gamma, double eps,
                  int act, double* o) {
    if (P < 0 || d <= 0 || eps < 0.0 || act < 0 || act > 2) return -1;
    for (int p = 0; p < P; ++p) {
        const float* yr = y + (size_t)p * d;
        const float* gr = g ? g + (size_t)p * d : NULL;
        double ss = 0.0;
        for (int c = 0; c < d; ++c) ss += (double)yr[c] * (double)yr[c];
        double inv = 1.0 / sqrt(ss / d + eps);
        for (int c = 0; c < d; ++c) {
            double f = 1.0;
            if (act != 0) {
                double x = (double)gr[c];
                double sg = 1.0 / (1.0 + exp(-x));
                f = act == 1 ? x * sg : sg;
            }
            o[(size_t)p * d + c] = (double)yr[c] * inv * (double)gamma[c] * f;
        }
    }
    return 0;
}
