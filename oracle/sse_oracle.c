/*
 * Plain fp64 CPU oracle for Sparse State Expansion (SSE): gated top-k routing
 * over N state partitions plus one always-active shared partition, with
 * GLA-style diagonal decay that advances only on visits.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this code; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source with the HIP library.
 *
 * Sources (reading slides "Scaling Linear Attention with Sparse State
 * Expansion"):
 *   - slide "A key vector decides where information is written", Eq. (6):
 *     S_t = Lambda_t S_{t-1} + phi(k_t)^T v_t, diagonal Lambda for GLA.
 *   - slide "One gate controls both writes and reads", Eqs. (9)-(14):
 *     e_t = softmax(x W_e), T_t = TopKIndices(e_t, k);
 *     S^i_t = Lambda_t S^i_{t-1} + e^i_t k_t^T v_t for i in T_t, else unchanged;
 *     o_t = sum_{i in T_t} e^i_t q_t S^i_t.
 *   - slide "SSE routes tokens into shared-parameter state partitions":
 *     one always-active shared partition.
 *   - slide "A memory decays only when its partition is visited" and slide
 *     "Varlen groups tokens while preserving causal order" (masking must also
 *     freeze inactive decay).
 *   - backup slide "Selected gate mass is usually below one": the selected
 *     softmax values are not renormalised.
 *
 * Readings (listed in the design notes):
 *   - selection is the top-k of the fp32 logits (same order as the softmax),
 *     ties to the lowest partition index; e is the fp64 softmax of all N logits;
 *   - Lambda_t is one decay per state row (key channel), applied on the left;
 *   - the shared partition (index N) is updated every token with weight 1,
 *     the same Lambda_t, and its own key/query (q_sh, k_sh; the caller passes
 *     q, k when there is no separate projection);  PARITY UNPINNED: the slides
 *     omit the shared partition's formula, so no printed value fixes it.
 *   - the output sums the routed contributions in rank order, then the shared one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* top-k of n logits by (value desc, index asc); writes k indices in rank order */
static void topk_logits(const float* g, int n, int k, int32_t* out) {
    unsigned char taken[256];
    memset(taken, 0, sizeof(taken));
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int i = 0; i < n; ++i) {
            if (taken[i]) continue;
            if (best < 0 || g[i] > g[best]) best = i; /* strict '>' keeps the lowest index on ties */
        }
        taken[best] = 1;
        out[r] = best;
    }
}

/*
 *   logits : [B,T,H,N] fp32 gate logits
 *   q, k   : [B,T,H,c] (k already softmax-normalised over c by the caller)
 *   v      : [B,T,H,d]
 *   lam    : [B,T,H,c] per-row decay in (0,1]
 *   q_sh, k_sh : [B,T,H,c] shared-partition query/key, or NULL to reuse q, k
 *   S      : [B,H,N+1,c,d] states, in/out (index N is the shared partition)
 *   o      : [B,T,H,d]
 *   sel    : [B,T,H,topk] selected partitions (optional, may be NULL)
 *   e_sel  : [B,T,H,topk] their softmax gate values (optional)
 *   masking: 0 = per-token definition above; 1 = the masking execution
 *            (every partition is visited, inactive ones with write/read weight
 *            0 and decay frozen to 1) -- a second algorithm for the same result.
 */
int orc_sse(int B, int T, int H, int N, int topk, int c, int d, const float* logits, const float* q,
            const float* k, const float* v, const float* lam, const float* q_sh, const float* k_sh,
            double* S, double* o, int32_t* sel, double* e_sel, int masking) {
    if (B < 0 || T < 0 || H <= 0 || N <= 0 || N > 256 || topk <= 0 || topk > N || c <= 0 || d <= 0)
        return -1;
    if (!q_sh) q_sh = q;
    if (!k_sh) k_sh = k;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            double* st = S + ((size_t)b * H + h) * (size_t)(N + 1) * c * d;
            double* e = (double*)malloc(sizeof(double) * N);
            int32_t* pick = (int32_t*)malloc(sizeof(int32_t) * topk);
            for (int t = 0; t < T; ++t) {
                size_t bth = ((size_t)b * T + t) * H + h;
                const float* g = logits + bth * N;
                const float* qt = q + bth * c;
                const float* kt = k + bth * c;
                const float* qs = q_sh + bth * c;
                const float* ks = k_sh + bth * c;
                const float* vt = v + bth * d;
                const float* lt = lam + bth * c;
                /* router: softmax over all N logits, hard top-k, no renormalisation */
                double mx = g[0];
                for (int i = 1; i < N; ++i)
                    if (g[i] > mx) mx = g[i];
                double z = 0.0;
                for (int i = 0; i < N; ++i) z += exp((double)g[i] - mx);
                for (int i = 0; i < N; ++i) e[i] = exp((double)g[i] - mx) / z;
                topk_logits(g, N, topk, pick);
                if (sel)
                    for (int r = 0; r < topk; ++r) sel[bth * topk + r] = pick[r];
                if (e_sel)
                    for (int r = 0; r < topk; ++r) e_sel[bth * topk + r] = e[pick[r]];
                double* ot = o + bth * d;
                for (int x = 0; x < d; ++x) ot[x] = 0.0;
                if (!masking) {
                    /* routed partitions in rank order: decay, gated write, gated read */
                    for (int r = 0; r < topk; ++r) {
                        int i = pick[r];
                        double* si = st + (size_t)i * c * d;
                        for (int row = 0; row < c; ++row)
                            for (int x = 0; x < d; ++x)
                                si[(size_t)row * d + x] = (double)lt[row] * si[(size_t)row * d + x] +
                                                          e[i] * (double)kt[row] * (double)vt[x];
                        for (int row = 0; row < c; ++row)
                            for (int x = 0; x < d; ++x)
                                ot[x] += e[i] * (double)qt[row] * si[(size_t)row * d + x];
                    }
                } else {
                    /* masking: replicate over every partition, mask inactive writes and
                     * reads, and freeze inactive decay (decay factor exactly 1) */
                    for (int i = 0; i < N; ++i) {
                        int active = 0;
                        for (int r = 0; r < topk; ++r) active |= (pick[r] == i);
                        double m = active ? 1.0 : 0.0;
                        double* si = st + (size_t)i * c * d;
                        for (int row = 0; row < c; ++row) {
                            double dec = active ? (double)lt[row] : 1.0;
                            for (int x = 0; x < d; ++x)
                                si[(size_t)row * d + x] = dec * si[(size_t)row * d + x] +
                                                          m * e[i] * (double)kt[row] * (double)vt[x];
                        }
                        if (active)
                            for (int row = 0; row < c; ++row)
                                for (int x = 0; x < d; ++x)
                                    ot[x] += e[i] * (double)qt[row] * si[(size_t)row * d + x];
                    }
                }
                /* shared partition: every token, weight 1 */
                double* ss = st + (size_t)N * c * d;
                for (int row = 0; row < c; ++row)
                    for (int x = 0; x < d; ++x)
                        ss[(size_t)row * d + x] = (double)lt[row] * ss[(size_t)row * d + x] +
                                                  (double)ks[row] * (double)vt[x];
                for (int row = 0; row < c; ++row)
                    for (int x = 0; x < d; ++x) ot[x] += (double)qs[row] * ss[(size_t)row * d + x];
            }
            free(e);
            free(pick);
        }
    return 0;
}
