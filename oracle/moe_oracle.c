/*
 * Oracle for the paged fused-MoE layer: plain, slow, obviously correct CPU code.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP path; the two meet only in the seeded inputs.
 *
 * Every floating-point result is accumulated in double precision from exact
 * widenings of the bf16 / fp32 inputs.  No blocking, no fusion, no reordering
 * beyond what the definitions below state.
 *
 * Source: "Rimuru: Unified Memory Management for Modern LLM Serving via Elastic
 * Expert Offloading" (paper-daily.com digest, English page), sections
 *   [K] "Expert weights are scattered across pages. How does the kernel read
 *       them?" -- the address formula addr_e(n,t), W1/W3 chosen by which half of
 *       the output columns n falls in, the per-expert location metadata (a page
 *       number for a cached expert, a buffer slot for one just copied in);
 *   [A] "The adjuster: when to evict an expert, and which one?" -- an expert
 *       is three pages: W1 (gate), W3 (up) and W2 (down);
 *   [P] "The pipeline: what happens in one scheduling round", step 5 -- the
 *       actual routing decides which experts a layer computes.
 * The pages do not print the routing rule, the token alignment, the W2 page
 * layout, the load-buffer slot layout or a worked numeric example of a layer;
 * the readings taken for each are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* exact widening of a bfloat16 bit pattern */
static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return (double)v;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Top-k softmax routing.  For each token t (row of the fp32 logits [T][E]):
 *   - pick k experts, largest logit first; equal logits go to the lower id;
 *   - weight of pick j: exp(l_j - l_max) / sum over the k picks of exp(l_i - l_max),
 *     i.e. the softmax renormalised over the chosen k;
 *   - with S = 1 a shared expert (id E) is appended as pick k with weight 1.
 * Selection compares the fp32 logits themselves, so the indices do not depend
 * on how exp is rounded.  Outputs: ids [T][k+S], w [T][k+S] (double).
 * Returns 0, or -1 for bad sizes.
 */
int oracle_route(const float *logits, int64_t T, int E, int k, int S,
                 int32_t *ids, double *w)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E || S < 0 || S > 1)
        return -1;
    const int keff = k + S;
    char *taken = (char *)malloc((size_t)E);
    if (!taken)
        return -1;
    for (int64_t t = 0; t < T; t++) {
        const float *row = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || row[e] > row[best])
                    best = e;
            }
            taken[best] = 1;
            ids[t * keff + j] = best;
        }
        double lmax = (double)row[ids[t * keff]];
        double denom = 0.0;
        for (int j = 0; j < k; j++)
            denom += exp((double)row[ids[t * keff + j]] - lmax);
        for (int j = 0; j < k; j++)
            w[t * keff + j] = exp((double)row[ids[t * keff + j]] - lmax) / denom;
        if (S) {
            ids[t * keff + k] = E;
            w[t * keff + k] = 1.0;
        }
    }
    free(taken);
    return 0;
}

/*
 * Token alignment for the grouped GEMMs (a stable counting sort of the flat
 * (token, pick) indices i = t*(k+S) + j by expert, each expert's segment padded
 * up to a multiple of the GEMM tile height BM):
 *   c_e = number of i with ids[i] == e,  P_e = ceil(c_e / BM) * BM,
 *   O_e = P_0 + ... + P_{e-1}  (experts in ascending id),
 *   sorted_ids[O_e + r] = the r-th smallest i routed to e, for r < c_e,
 *   sorted_ids[O_e + r] = n (sentinel) for c_e <= r < P_e,
 *   block_expert[b] = e for every BM-row block b inside e's segment,
 *   num_padded = sum of P_e.
 * Experts with no tokens get no block.  Returns 0, -1 for a bad id or size,
 * -2 when an output capacity is too small.
 */
int oracle_align(const int32_t *ids, int64_t n, int E_tot, int BM,
                 int32_t *sorted_ids, int64_t sorted_cap,
                 int32_t *block_expert, int64_t blocks_cap, int32_t *num_padded)
{
    if (n < 0 || E_tot <= 0 || BM <= 0)
        return -1;
    int64_t *count = (int64_t *)calloc((size_t)E_tot, sizeof(int64_t));
    int64_t *offset = (int64_t *)calloc((size_t)E_tot, sizeof(int64_t));
    int64_t *cursor = (int64_t *)calloc((size_t)E_tot, sizeof(int64_t));
    int rc = 0;
    if (!count || !offset || !cursor) {
        rc = -1;
        goto out;
    }
    for (int64_t i = 0; i < n; i++) {
        if (ids[i] < 0 || ids[i] >= E_tot) {
            rc = -1;
            goto out;
        }
        count[ids[i]]++;
    }
    int64_t total = 0;
    for (int e = 0; e < E_tot; e++) {
        int64_t padded = (count[e] + BM - 1) / BM * BM;
        offset[e] = total;
        total += padded;
    }
    if (total > sorted_cap || total / BM > blocks_cap) {
        rc = -2;
        goto out;
    }
    for (int e = 0; e < E_tot; e++)
        cursor[e] = offset[e];
    for (int64_t i = 0; i < n; i++)
        sorted_ids[cursor[ids[i]]++] = (int32_t)i;
    for (int e = 0; e < E_tot; e++) {
        int64_t end = offset[e] + (count[e] + BM - 1) / BM * BM;
        for (int64_t pos = cursor[e]; pos < end; pos++)
            sorted_ids[pos] = (int32_t)n;
        for (int64_t b = offset[e] / BM; b < end / BM; b++)
            block_expert[b] = e;
    }
    *num_padded = (int32_t)total;
out:
    free(count);
    free(offset);
    free(cursor);
    return rc;
}

/*
 * Element address of one weight, [K] address formula:
 *     addr_e(n, t) = B_P + p_e(n)*f*d + (n mod f)*d + t
 * for the fused gate/up operand (which = 0): n in [0, 2f) is the output column,
 * t in [0, d) the offset along the hidden dimension, p_e(n) the W1 page when
 * n < f and the W3 page otherwise.
 * Readings where the pages are silent:
 *   - the down projection (which = 1) is a page [d rows][f] like W1/W3:
 *     addr = B_P + p_e(W2)*f*d + r*f + c, r in [0, d), c in [0, f);
 *   - an expert just copied in sits in load-buffer slot s with its three
 *     matrices back to back, so the same formula holds with B_P replaced by the
 *     active buffer's base and the page number replaced by 3s + m
 *     (m = 0 W1, 1 W3, 2 W2);
 *   - units are bf16 elements.
 * locs is [E_tot][4] int32: kind (0 pool, 1 load buffer), then the W1, W3, W2
 * pages (pool) or the slot (load buffer).
 * Output: *base = 0 for the pool, 1 + active_buf for a load buffer; *off =
 * element offset from that base.  Returns 0, or -1 for an argument out of range.
 */
int oracle_addr(const int32_t *locs, int E_tot, int64_t f, int64_t d,
                int64_t num_pages, int slots, int active_buf,
                int e, int which, int64_t row, int64_t col,
                int64_t *off, int32_t *base)
{
    if (e < 0 || e >= E_tot || (which != 0 && which != 1))
        return -1;
    if (which == 0 && (row < 0 || row >= 2 * f || col < 0 || col >= d))
        return -1;
    if (which == 1 && (row < 0 || row >= d || col < 0 || col >= f))
        return -1;
    const int32_t *L = locs + 4 * e;
    int64_t page;
    if (L[0] == 0) {
        page = which == 0 ? (row < f ? L[1] : L[2]) : L[3];
        if (page < 0 || page >= num_pages)
            return -1;
        *base = 0;
    } else if (L[0] == 1) {
        if (L[1] < 0 || L[1] >= slots || active_buf < 0 || active_buf > 1)
            return -1;
        int m = which == 0 ? (row < f ? 0 : 1) : 2;
        page = 3 * (int64_t)L[1] + m;
        *base = 1 + active_buf;
    } else {
        return -1;
    }
    if (which == 0)
        *off = page * f * d + (row % f) * d + col;
    else
        *off = page * f * d + row * f + col;
    return 0;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/*
 * The MoE layer output for the listed tokens, straight from its definition on
 * contiguous weights:
 *     y_t = sum_j w_{t,j} * FFN_{e_{t,j}}(x_t),
 *     FFN_e(x) = W2_e (silu(W1_e x) * (W3_e x)),   silu(g) = g / (1 + e^-g),
 * with W1 = gate and W3 = up ([K]: "gate and up ... W1, W3" in that order;
 * [A]: W2 is the down projection).  The shared expert, when present, is just
 * one more (id, weight 1) pick.
 * x [T][d], w13 [E_tot][2f][d] (rows [0,f) W1, [f,2f) W3), w2 [E_tot][d][f]:
 * bf16 bits.  ids, w: [T][keff].  tokens: ntok token indices; y [ntok][d].
 * Returns 0, or -1 for a bad id.
 */
int oracle_moe(const uint16_t *x, const uint16_t *w13, const uint16_t *w2,
               const int32_t *ids, const double *w, int64_t T, int64_t d,
               int64_t f, int E_tot, int keff, const int64_t *tokens,
               int64_t ntok, double *y)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t q = 0; q < ntok; q++) {
        int64_t t = tokens[q];
        double *xr = (double *)malloc((size_t)d * sizeof(double));
        double *act = (double *)malloc((size_t)f * sizeof(double));
        double *yr = y + q * d;
        for (int64_t r = 0; r < d; r++)
            yr[r] = 0.0;
        if (t < 0 || t >= T || !xr || !act) {
            bad = 1;
            free(xr);
            free(act);
            continue;
        }
        for (int64_t i = 0; i < d; i++)
            xr[i] = bf16_value(x[t * d + i]);
        for (int j = 0; j < keff; j++) {
            int e = ids[t * keff + j];
            if (e < 0 || e >= E_tot) {
                bad = 1;
                break;
            }
            const uint16_t *W1 = w13 + (int64_t)e * 2 * f * d;
            const uint16_t *W3 = W1 + f * d;
            const uint16_t *W2 = w2 + (int64_t)e * d * f;
            for (int64_t c = 0; c < f; c++) {
                double g = 0.0, u = 0.0;
                for (int64_t i = 0; i < d; i++) {
                    g += xr[i] * bf16_value(W1[c * d + i]);
                    u += xr[i] * bf16_value(W3[c * d + i]);
                }
                act[c] = silu(g) * u;
            }
            double wt = w[t * keff + j];
            for (int64_t r = 0; r < d; r++) {
                double o = 0.0;
                for (int64_t c = 0; c < f; c++)
                    o += act[c] * bf16_value(W2[r * f + c]);
                yr[r] += wt * o;
            }
        }
        free(xr);
        free(act);
    }
    return bad ? -1 : 0;
}
