/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the routed
 * Mixture-of-Experts SwiGLU expert FFN with intra-expert activation sparsity.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load or call this file.  It shares no code, header, table or helper with the
 * GPU library, and the GPU library never calls it.
 *
 * Every floating-point quantity is computed in double precision from the
 * exact values of the inputs (bf16 and fp32 inputs upcast exactly).  There is
 * no blocking, fusion or reordering: each output is the definition written out
 * as nested loops in the order the method states its steps.
 *
 * Sources (all describe arXiv 2605.08575, "Uncovering Intra-expert Activation
 * Sparsity for Efficient Mixture-of-Expert Model Execution"):
 *   [TS]  gist.science explanation page, "Technical Summary" -- subsections
 *         Methodology (Gate Projection, Activation Masking, Fused Up-Down
 *         Projection, Dynamic Switching) and Results.
 *   [LAY] the same page's lay explanation, "How They Did It: The Skip-List
 *         System".
 *   [ABS] mlsanity.com page, "Abstract (arXiv)".
 *   Readings where the pages are silent are marked READING and are listed in
 *   the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ----------------------------------------------------------------------- */
/* Input decoding: bf16 is the upper half of an IEEE binary32, so widening   */
/* is exact.                                                                 */
/* ----------------------------------------------------------------------- */
static double load_elem(const void *base, int is_bf16, size_t i)
{
    if (is_bf16) {
        uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

/* NaN logits take part in ranking as -infinity (READING: the pages keep the
 * router unchanged and do not define non-finite logits). */
static double rank_value(float v)
{
    return isnan(v) ? -INFINITY : (double)v;
}

/* ----------------------------------------------------------------------- */
/* Step 1: routing.  [TS] Methodology keeps the router logic unchanged; the  */
/* router is the standard softmax over all routed experts followed by top-K. */
/* Softmax is strictly increasing, so the K most probable experts are the K  */
/* largest logits; the ranking is taken on the raw fp32 logits so that no    */
/* rounding of exp() can create a tie.  Ties go to the lower expert id.      */
/* Slots are in descending-probability order.                                */
/* ----------------------------------------------------------------------- */
int oracle_route(const float *logits, int T, int E, int K, int renormalize,
                 int32_t *ids, double *w)
{
    if (T < 0 || E <= 0 || K <= 0 || K > E) return 1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken) return 2;
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || rank_value(l[e]) > rank_value(l[best])) best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * K + k] = best;
        }
        /* softmax over all E experts, shifted by the maximum for range */
        double m = -INFINITY;
        for (int e = 0; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double denom = 0.0;
        for (int e = 0; e < E; ++e) denom += exp((double)l[e] - m);
        double sel = 0.0;
        for (int k = 0; k < K; ++k) {
            double p = exp((double)l[ids[(size_t)t * K + k]] - m) / denom;
            w[(size_t)t * K + k] = p;
            sel += p;
        }
        if (renormalize)
            for (int k = 0; k < K; ++k) w[(size_t)t * K + k] /= sel;
    }
    free(taken);
    return 0;
}

/* SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)).  The activation score of a
 * neuron is computed from the gate projection alone ([TS] Gate Projection). */
static double silu(double g)
{
    return g / (1.0 + exp(-g));
}

/* Geometry of one expert: routed experts 0..E-1 use (w_gate, w_up, w_down)
 * with I rows, shared experts E..E+S-1 use (ws_*) with I_shared rows.  All
 * three matrices are neuron-major [rows, H]: row j of the down matrix holds
 * neuron j's output weights (the transpose of the usual [H, I] layout). */
typedef struct {
    const void *g, *u, *d;
    int rows;
} expert_view;

static expert_view expert_at(int e, int E, int I, int Is, int H, int bf16,
                             const void *wg, const void *wu, const void *wd,
                             const void *swg, const void *swu, const void *swd)
{
    expert_view v;
    size_t esz = bf16 ? 2 : 4;
    if (e < E) {
        size_t off = (size_t)e * I * H * esz;
        v.g = (const char *)wg + off;
        v.u = (const char *)wu + off;
        v.d = (const char *)wd + off;
        v.rows = I;
    } else {
        size_t off = (size_t)(e - E) * Is * H * esz;
        v.g = (const char *)swg + off;
        v.u = (const char *)swu + off;
        v.d = (const char *)swd + off;
        v.rows = Is;
    }
    return v;
}

/*
 * oracle_moe -- the layer output and the active-neuron masks.
 *
 * For every token t and slot k (routed slots 0..K-1 from oracle_route, then
 * the S shared experts in slots K..K+S-1 with weight 1, READING for shared
 * experts: [TS] Methodology says they are always active):
 *   g_j  = sum_h x[t,h] * Wgate[e][j,h]           ([TS] Gate Projection: dense)
 *   a_j  = SiLU(g_j)                              (the activation score)
 *   m_j  = NOT(|a_j| < tau_e)                     ([TS] Activation Masking:
 *                                                  one elementwise threshold;
 *                                                  READING: equality and NaN
 *                                                  count as active)
 *   u_j  = sum_h x[t,h] * Wup[e][j,h]   only where m_j = 1
 *   h_j  = a_j * u_j where m_j = 1, exactly 0 otherwise ([LAY] Skip-List: an
 *          inactive neuron's weights are never touched)
 *   o    = sum_{j : m_j = 1} h_j * Wdown[e][j,:]  ([TS] Fused Up-Down
 *                                                  Projection)
 *   y_t  = sum_{k<K} w[t,k] * o_{t,k} + sum_{s<S} o_{t,K+s}
 * dense != 0 sets m_j = 1 everywhere (the ordinary dense SwiGLU MoE layer).
 * force_mask, when non-NULL, supplies m directly (same layout as mask_bits).
 *
 * Layouts: x [T,H]; logits [T,E] fp32; weights neuron-major [E,I,H] and
 * [S,I_shared,H]; tau [E+S]; y [T,H]; mask_bits [T,K+S,W] with
 * W = ceil(max(I,I_shared)/32), bit j%32 of word j/32; scores [T,K+S,Imax];
 * union_idx [E+S,Imax] (first union_cnt[e] entries, ascending);
 * ids [T,K]; w [T,K].  Every output pointer except y may be NULL.
 */
int oracle_moe(int T, int H, int E, int I, int K, int S, int Is,
               int renormalize, int bf16, const void *x, const float *logits,
               const void *wg, const void *wu, const void *wd,
               const void *swg, const void *swu, const void *swd,
               const double *tau, int dense, const uint32_t *force_mask,
               double *y, uint32_t *mask_bits, double *scores,
               int32_t *union_idx, int32_t *union_cnt,
               int32_t *ids_out, double *w_out, int threads)
{
    if (T < 0 || H <= 0 || E <= 0 || I <= 0 || K <= 0 || K > E || S < 0) return 1;
    if (S > 0 && Is <= 0) return 1;
    const int slots = K + S;
    const int Imax = (S > 0 && Is > I) ? Is : I;
    const int W = (Imax + 31) / 32;

    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1) * K);
    double *w = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * K);
    uint32_t *mbits = (uint32_t *)calloc((size_t)(T > 0 ? T : 1) * slots * W, sizeof(uint32_t));
    if (!ids || !w || !mbits) { free(ids); free(w); free(mbits); return 2; }
    oracle_route(logits, T, E, K, renormalize, ids, w);

    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1)
    for (int t = 0; t < T; ++t) {
        double *o = (double *)malloc(sizeof(double) * (size_t)H);
        if (!o) { failed = 1; continue; }
        for (int c = 0; c < H; ++c) y[(size_t)t * H + c] = 0.0;
        for (int k = 0; k < slots; ++k) {
            const int e = (k < K) ? ids[(size_t)t * K + k] : E + (k - K);
            const double weight = (k < K) ? w[(size_t)t * K + k] : 1.0;
            const expert_view v = expert_at(e, E, I, Is, H, bf16, wg, wu, wd, swg, swu, swd);
            const double tau_e = tau ? tau[e] : 0.0;
            uint32_t *mrow = mbits + ((size_t)t * slots + k) * W;
            for (int c = 0; c < H; ++c) o[c] = 0.0;
            for (int j = 0; j < v.rows; ++j) {
                /* gate projection and score */
                double g = 0.0;
                for (int hh = 0; hh < H; ++hh)
                    g += load_elem(x, bf16, (size_t)t * H + hh) *
                         load_elem(v.g, bf16, (size_t)j * H + hh);
                const double a = silu(g);
                if (scores) scores[((size_t)t * slots + k) * Imax + j] = a;
                /* threshold mask */
                int m;
                if (force_mask)
                    m = (int)((force_mask[((size_t)t * slots + k) * W + j / 32] >> (j % 32)) & 1u);
                else if (dense)
                    m = 1;
                else
                    m = !(fabs(a) < tau_e);
                if (!m) continue;
                mrow[j / 32] |= 1u << (j % 32);
                /* up projection of an active neuron only */
                double u = 0.0;
                for (int hh = 0; hh < H; ++hh)
                    u += load_elem(x, bf16, (size_t)t * H + hh) *
                         load_elem(v.u, bf16, (size_t)j * H + hh);
                const double hval = a * u;
                /* down projection: neuron j's output row, scaled by h_j */
                for (int c = 0; c < H; ++c)
                    o[c] += hval * load_elem(v.d, bf16, (size_t)j * H + c);
            }
            for (int c = 0; c < H; ++c) y[(size_t)t * H + c] += weight * o[c];
        }
        free(o);
    }

    if (!failed) {
        if (mask_bits) memcpy(mask_bits, mbits, sizeof(uint32_t) * (size_t)T * slots * W);
        if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * K);
        if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)T * K);
        /* Per-expert union of active neurons over every (token, slot) pair the
         * expert serves; listed in ascending neuron order. */
        if (union_idx || union_cnt) {
            uint32_t *ubits = (uint32_t *)calloc((size_t)(E + S) * W, sizeof(uint32_t));
            if (!ubits) {
                failed = 1;
            } else {
                for (int t = 0; t < T; ++t)
                    for (int k = 0; k < slots; ++k) {
                        const int e = (k < K) ? ids[(size_t)t * K + k] : E + (k - K);
                        for (int q = 0; q < W; ++q)
                            ubits[(size_t)e * W + q] |= mbits[((size_t)t * slots + k) * W + q];
                    }
                for (int e = 0; e < E + S; ++e) {
                    const int rows = (e < E) ? I : Is;
                    int cnt = 0;
                    for (int j = 0; j < rows; ++j) {
                        if (!((ubits[(size_t)e * W + j / 32] >> (j % 32)) & 1u)) continue;
                        if (union_idx) union_idx[(size_t)e * Imax + cnt] = j;
                        ++cnt;
                    }
                    if (union_cnt) union_cnt[e] = cnt;
                }
                free(ubits);
            }
        }
    }
    free(ids);
    free(w);
    free(mbits);
    return failed ? 2 : 0;
}

/* ----------------------------------------------------------------------- */
/* Step 9 (off the timed path): threshold calibration to a target sparsity. */
/* [TS] Results speaks of sparsity cutoffs and a target sparsity; READING:  */
/* tau is the order statistic v[floor(q*N)] (0-indexed) of the ascending    */
/* population v of |SiLU(gate)| scores, so that exactly floor(q*N) scores   */
/* fall strictly below tau when there are no ties.  q = 0 gives tau = 0 and */
/* floor(q*N) = N gives +infinity.  NaN scores sort after +infinity.        */
/* ----------------------------------------------------------------------- */
static int cmp_score(const void *pa, const void *pb)
{
    const double a = *(const double *)pa, b = *(const double *)pb;
    const int na = isnan(a), nb = isnan(b);
    if (na || nb) return na - nb;
    return (a > b) - (a < b);
}

static double order_statistic(double *v, long n, double q)
{
    if (q == 0.0) return 0.0;
    const long kappa = (long)floor(q * (double)n);
    if (kappa >= n) return INFINITY;
    qsort(v, (size_t)n, sizeof(double), cmp_score);
    return v[kappa];
}

/*
 * oracle_calibrate -- tau per expert [E+S].
 * Population ([TS] Methodology, "within active experts"; routed and shared
 * experts are treated separately): |a_j| for every calibration token t, every
 * routed slot k < K and every neuron j of the selected expert.  The S shared
 * experts form their own population over all tokens.  per_expert != 0 takes
 * the order statistic per expert over that expert's own pairs and falls back
 * to the routed population's tau for a routed expert with no pairs.
 * q must lie in [0, 1].  The q value is the caller's float widened exactly.
 */
int oracle_calibrate(int Tc, int H, int E, int I, int K, int S, int Is,
                     int bf16, const void *x, const float *logits,
                     const void *wg, const void *swg, double q, int per_expert,
                     double *tau_out, int threads)
{
    if (Tc <= 0 || H <= 0 || E <= 0 || I <= 0 || K <= 0 || K > E || S < 0) return 1;
    if (S > 0 && Is <= 0) return 1;
    if (!(q >= 0.0 && q <= 1.0)) return 1;
    const int slots = K + S;
    const int Imax = (S > 0 && Is > I) ? Is : I;
    double *sc = (double *)malloc(sizeof(double) * (size_t)Tc * slots * Imax);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)Tc * K);
    double *wts = (double *)malloc(sizeof(double) * (size_t)Tc * K);
    if (!sc || !ids || !wts) { free(sc); free(ids); free(wts); return 2; }
    oracle_route(logits, Tc, E, K, 1, ids, wts);

    /* score of every neuron of every expert a calibration token is sent to */
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1)
    for (int t = 0; t < Tc; ++t)
        for (int k = 0; k < slots; ++k) {
            const int e = (k < K) ? ids[(size_t)t * K + k] : E + (k - K);
            const expert_view v = expert_at(e, E, I, Is, H, bf16, wg, wg, wg, swg, swg, swg);
            for (int j = 0; j < v.rows; ++j) {
                double g = 0.0;
                for (int hh = 0; hh < H; ++hh)
                    g += load_elem(x, bf16, (size_t)t * H + hh) *
                         load_elem(v.g, bf16, (size_t)j * H + hh);
                sc[((size_t)t * slots + k) * Imax + j] = silu(g);
            }
        }

    double *pop = (double *)malloc(sizeof(double) * ((size_t)Tc * K * I + (size_t)Tc * (S > 0 ? Is : 0) * (S > 0 ? S : 0) + 1));
    if (!pop) { free(sc); free(ids); free(wts); return 2; }

    /* routed population */
    long n = 0;
    for (int t = 0; t < Tc; ++t)
        for (int k = 0; k < K; ++k)
            for (int j = 0; j < I; ++j)
                pop[n++] = fabs(sc[((size_t)t * slots + k) * Imax + j]);
    const double tau_routed = order_statistic(pop, n, q);
    /* shared population */
    double tau_shared = 0.0;
    if (S > 0) {
        n = 0;
        for (int t = 0; t < Tc; ++t)
            for (int k = K; k < slots; ++k)
                for (int j = 0; j < Is; ++j)
                    pop[n++] = fabs(sc[((size_t)t * slots + k) * Imax + j]);
        tau_shared = order_statistic(pop, n, q);
    }
    for (int e = 0; e < E; ++e) tau_out[e] = tau_routed;
    for (int s = 0; s < S; ++s) tau_out[E + s] = tau_shared;

    if (per_expert) {
        for (int e = 0; e < E; ++e) {
            n = 0;
            for (int t = 0; t < Tc; ++t)
                for (int k = 0; k < K; ++k) {
                    if (ids[(size_t)t * K + k] != e) continue;
                    for (int j = 0; j < I; ++j)
                        pop[n++] = fabs(sc[((size_t)t * slots + k) * Imax + j]);
                }
            tau_out[e] = (n > 0) ? order_statistic(pop, n, q) : tau_routed;
        }
        for (int s = 0; s < S; ++s) {
            n = 0;
            for (int t = 0; t < Tc; ++t)
                for (int j = 0; j < Is; ++j)
                    pop[n++] = fabs(sc[((size_t)t * slots + K + s) * Imax + j]);
            tau_out[E + s] = order_statistic(pop, n, q);
        }
    }
    free(pop);
    free(sc);
    free(ids);
    free(wts);
    return 0;
}

/* ----------------------------------------------------------------------- */
/* The top-k alternative to the threshold.  [TS] Methodology, Activation    */
/* Masking: the method masks with one elementwise threshold pass instead of */
/* selecting the top-k activations per token.  For comparison, this takes   */
/* that alternative literally: for each (token, slot) pair the `budget`     */
/* neurons of largest |a_j| are active.  READING (the pages give no tie     */
/* rule): a NaN score ranks first, as the threshold counts NaN as active,   */
/* and equal scores go to the lower neuron index.  An expert with at most   */
/* `budget` rows keeps them all.                                            */
/* ----------------------------------------------------------------------- */
typedef struct {
    double mag;  /* |a_j| */
    int j;
} ranked_neuron;

/* Descending |a| with NaN first; equal magnitudes by ascending j. */
static int cmp_ranked(const void *pa, const void *pb)
{
    const ranked_neuron *a = (const ranked_neuron *)pa, *b = (const ranked_neuron *)pb;
    const int na = isnan(a->mag), nb = isnan(b->mag);
    if (na != nb) return nb - na;
    if (!na) {
        if (a->mag > b->mag) return -1;
        if (a->mag < b->mag) return 1;
    }
    return (a->j > b->j) - (a->j < b->j);
}

/*
 * oracle_topk_mask -- mask words [npairs, W] (W = ceil(Imax/32)) from the
 * scores a [npairs, Imax] of oracle_moe; rows[p] is the row count of pair p's
 * expert.  Returns 0, or 1 for invalid arguments.
 */
int oracle_topk_mask(int npairs, int Imax, const double *scores, const int32_t *rows, int budget,
                     uint32_t *mask)
{
    if (npairs < 0 || Imax <= 0 || budget < 0 || !scores || !rows || !mask) return 1;
    const int W = (Imax + 31) / 32;
    ranked_neuron *v = (ranked_neuron *)malloc(sizeof(ranked_neuron) * (size_t)Imax);
    if (!v) return 1;
    for (int p = 0; p < npairs; ++p) {
        uint32_t *m = mask + (size_t)p * W;
        for (int w = 0; w < W; ++w) m[w] = 0u;
        const int n = rows[p];
        if (n < 0 || n > Imax) {
            free(v);
            return 1;
        }
        for (int j = 0; j < n; ++j) {
            v[j].mag = fabs(scores[(size_t)p * Imax + j]);
            v[j].j = j;
        }
        qsort(v, (size_t)n, sizeof(ranked_neuron), cmp_ranked);
        const int keep = budget < n ? budget : n;
        for (int i = 0; i < keep; ++i) m[v[i].j / 32] |= 1u << (v[i].j % 32);
    }
    free(v);
    return 0;
}
