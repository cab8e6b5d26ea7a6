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
 * Parallel over (b,h) only; the token loop is the plain sequential order.
 */
int orc_sdm_recurrence(int B, int T, int H, long long N, int dv, int W, int R, int residual_mode,
                       const int32_t* idx_w, const double* wt_w, const int32_t* idx_r,
                       const double* wt_r, const float* v, const float* alpha, const float* beta,
                       double* M, double* y) {
    if (B < 0 || T < 0 || H <= 0 || N <= 0 || dv <= 0 || W <= 0 || R <= 0) return -1;
    if (residual_mode != 0 && residual_mode != 1) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
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
                    for (int c = 0; c < dv; ++c) mt[(size_t)n * dv + c] = a * tab[(size_t)iw[n] * dv + c];
                if (residual_mode == 0) {
                    for (int c = 0; c < dv; ++c) {
                        double s = 0.0;
                        for (int n = 0; n < W; ++n) s += gw[n] * mt[(size_t)n * dv + c];
                        vhat[c] = s;
                    }
                    for (int n = 0; n < W; ++n)
                        for (int c = 0; c < dv; ++c)
                            tab[(size_t)iw[n] * dv + c] =
                                mt[(size_t)n * dv + c] + be * gw[n] * ((double)vt[c] - vhat[c]);
                } else {
                    for (int n = 0; n < W; ++n)
                        for (int c = 0; c < dv; ++c)
                            tab[(size_t)iw[n] * dv + c] =
                                mt[(size_t)n * dv + c] +
                                be * gw[n] * ((double)vt[c] - mt[(size_t)n * dv + c]);
                }
                /* Eq. (5): read after writing */
                double* yt = y + bth * dv;
                for (int c = 0; c < dv; ++c) {
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
