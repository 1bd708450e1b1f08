/*
 * csa2_oracle.c -- plain, slow CPU oracle of the CSA2 sparse-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this code.  It shares no source with
 * the HIP library and the HIP library never calls it.
 *
 * What it follows (page "DeepSeek V4.1 Flash", k-a.in):
 *   - "Sparse attention" key fact: each query reads its Top-K main-KV entries
 *     plus a sliding window of recent tokens, not the whole context.
 *   - "Hierarchical indexer" key fact (and the forum summary's remark that the
 *     hierarchical sparse indexer narrows candidates down to blocks): a block
 *     pass keeps a bounded pool of blocks; only their tokens are scored.
 *   - "CSA2 with cross-layer reuse" mode table: Full computes fresh indices,
 *     Reindex uses its own indexer query over shared keys, Reuse takes the
 *     indices of an earlier layer; every mode has its own main Q and own
 *     sliding-window K/V.
 *   - the architecture figure's caption on the same page names CSA2(ratio,
 *     mode) with a compression ratio and defines neither the ratio nor the
 *     compressor.  Reading (orc_visible_entries): with ratio r, main-KV entry
 *     j stands for the r tokens j*r .. j*r + r - 1 and exists once its last
 *     token has arrived; the selection runs over entries, the window keeps one
 *     row per token.  The entries themselves arrive precomputed, like every
 *     other K/V row.
 * The pages leave the scores open.  The library fixes them as:
 *   - token score  s_p = <q_idx, k_idx[p]>            (int8 x int8, exact)
 *   - block score  s_j = <q_idx, round(mean of k_idx over block j)>
 * with the readings written next to each function below.
 *
 * Precision: integers are exact (int64); attention is fp64 on the exact input
 * values (fp32 or bf16 widened).
 *
 * Parity pins: every function here is pinned by tests against brute force,
 * closed forms or a hand-computed toy; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Element access: the attention inputs are either fp32 or bf16 bit patterns. */
/* ------------------------------------------------------------------------ */
enum { ORC_F32 = 0, ORC_BF16 = 1 };

static double load_elem(const void *base, int elem, size_t i)
{
    if (elem == ORC_F32)
        return (double)((const float *)base)[i];
    /* bf16: the upper 16 bits of an IEEE fp32 */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Step 1: block keys.                                                      */
/* ------------------------------------------------------------------------ */

/* sum / n rounded to the nearest integer, exact ties going to the even
 * neighbour (the rounding of the "int8-rounded mean"; the pages do not name a
 * rounding mode, round-half-even is the reading taken). */
int64_t orc_round_half_even_div(int64_t sum, int64_t n)
{
    int64_t q = sum / n, r = sum % n;        /* C truncates toward zero      */
    if (r < 0) { q -= 1; r += n; }           /* now q = floor(sum/n), 0<=r<n */
    if (2 * r > n) return q + 1;
    if (2 * r < n) return q;
    return (q % 2 == 0) ? q : q + 1;         /* exact tie: pick the even one */
}

/* Key of block j as seen by a query at position t: the per-dimension rounded
 * mean of the block's rows that are visible to the query (positions
 * j*B .. min(j*B+B-1, t)).  A block that is not yet full (only the query's own
 * block can be) therefore averages only the tokens that exist at time t.
 * (The whole-block tail reading passes t = T-1 here.)
 * k_seq is one sequence's indexer keys, row-major [T][d]. */
void orc_block_key(const int8_t *k_seq, int d, int B, int j, int t, int8_t *key)
{
    int first = j * B;
    int last = first + B - 1;
    if (last > t) last = t;
    int64_t n = last - first + 1;
    for (int c = 0; c < d; c++) {
        int64_t sum = 0;
        for (int p = first; p <= last; p++)
            sum += k_seq[(size_t)p * d + c];
        key[c] = (int8_t)orc_round_half_even_div(sum, n);
    }
}

static int64_t dot_i8(const int8_t *a, const int8_t *b, int d)
{
    int64_t s = 0;
    for (int c = 0; c < d; c++)
        s += (int64_t)a[c] * (int64_t)b[c];
    return s;
}

/* ------------------------------------------------------------------------ */
/* Steps 2-5: block pool and token Top-K for one query.                     */
/* ------------------------------------------------------------------------ */

typedef struct { int64_t score; int32_t id; } scored;

/* Total order used for every selection: higher score first; on equal scores
 * the lower position (or lower block id) wins. */
static int by_score_then_id(const void *pa, const void *pb)
{
    const scored *a = pa, *b = pb;
    if (a->score != b->score) return (a->score > b->score) ? -1 : 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

static int by_id(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* One query at position t of a sequence with indexer keys k_seq [T][d].
 *   blk_ids[P]: the pooled blocks in ascending order, -1 padded; *blk_cnt
 *   topk[K]   : the selected positions in ascending order, -1 padded; *topk_cnt
 * Pool (hierarchical pass): every block with at least one visible token is
 * eligible; if there are at most P of them all are kept, otherwise the P best
 * by (block score desc, block id asc).
 * Candidates: the visible positions (p <= t) of the pooled blocks.
 * Top-K: if there are at most K candidates all are kept, otherwise the K best
 * by (token score desc, position asc).
 * Returns 0, or -1 on bad arguments. */
/* Token Top-K of one query over a given pool (ascending block ids, n_pool
 * of them): the candidates are the positions p <= t of the pooled blocks,
 * scored <q_idx, k_idx[p]>; if there are more than K, the K best by (score
 * desc, position asc) are kept ("Sparse attention": Top-512 main-KV entries;
 * ties go to the lower position).  Output ascending, padded with -1. */
int orc_topk_one(const int8_t *q_idx, const int8_t *k_seq, int T, int t, int d, int B,
                 const int32_t *pool, int n_pool, int K, int32_t *topk, int32_t *topk_cnt)
{
    if (t < 0 || t >= T || d <= 0 || B <= 0 || K < 0 || n_pool < 0) return -1;
    scored *cand = malloc(sizeof(scored) * (size_t)(n_pool > 0 ? n_pool : 1) * (size_t)B);
    if (!cand) return -1;
    int n_cand = 0;
    for (int i = 0; i < n_pool; i++) {
        if (pool[i] < 0 || pool[i] > t / B) { free(cand); return -1; }
        for (int w = 0; w < B; w++) {
            int p = pool[i] * B + w;
            if (p > t) break;
            cand[n_cand].score = dot_i8(q_idx, k_seq + (size_t)p * d, d);
            cand[n_cand].id = p;
            n_cand++;
        }
    }
    int n_keep = n_cand;
    if (n_cand > K) {
        qsort(cand, (size_t)n_cand, sizeof(scored), by_score_then_id);
        n_keep = K;
    }
    int32_t *sel = malloc(sizeof(int32_t) * (size_t)(n_keep > 0 ? n_keep : 1));
    if (!sel) { free(cand); return -1; }
    for (int i = 0; i < n_keep; i++) sel[i] = cand[i].id;
    qsort(sel, (size_t)n_keep, sizeof(int32_t), by_id);
    for (int i = 0; i < K; i++) topk[i] = (i < n_keep) ? sel[i] : -1;
    *topk_cnt = n_keep;
    free(sel); free(cand);
    return 0;
}

/* Main-KV entries a query at token position t sees when every entry
 * compresses r consecutive tokens: entry j (tokens j*r .. j*r + r - 1) is
 * complete once (j + 1) * r - 1 <= t, i.e. for j + 1 <= (t + 1) / r, so the
 * visible entries are 0 .. (t + 1) / r - 1.  With r = 1 every entry is one
 * token and the count is t + 1.  Returns -1 for r < 1 or t < 0. */
int orc_visible_entries(int t, int r)
{
    if (r < 1 || t < 0) return -1;
    return (int)(((int64_t)t + 1) / r);   /* t + 1 may exceed INT32_MAX */
}

/* No visible entry: an empty selection (every slot -1, counts 0). */
static void empty_selection(int32_t *ids, int n, int32_t *cnt)
{
    for (int i = 0; i < n; i++) ids[i] = -1;
    *cnt = 0;
}

/* Token Top-K over given pools (blk_ids rows of P entries, blk_cnt counts)
 * for queries [q_begin, q_end): the Reindex variant that keeps the pool of
 * the shared index set and reruns only the token selection.  q_pos holds
 * token positions; with ratio r the candidates are the visible entries. */
int orc_topk_batch(int q_begin, int q_end, const int8_t *q_idx, const int32_t *q_seq,
                   const int32_t *q_pos, const int8_t *k_idx, int T, int d, int B, int P, int K,
                   int ratio, const int32_t *blk_ids, const int32_t *blk_cnt, int32_t *topk,
                   int32_t *topk_cnt)
{
    int bad = 0;
    for (int i = q_begin; i < q_end; i++) {
        const int s = q_seq[i];
        const int n_vis = orc_visible_entries(q_pos[i], ratio);
        if (n_vis < 0) { bad++; continue; }
        if (n_vis == 0) {
            if (blk_cnt[i] != 0) { bad++; continue; }
            empty_selection(topk + (size_t)i * K, K, topk_cnt + i);
            continue;
        }
        bad += orc_topk_one(q_idx + (size_t)i * d, k_idx + (size_t)s * T * d, T, n_vis - 1, d, B,
                            blk_ids + (size_t)i * P, blk_cnt[i], K, topk + (size_t)i * K, topk_cnt + i) != 0;
    }
    return bad;
}

/* The query's own block is partial when t is not its last position.  The
 * pages do not say how such a block enters the block pass; three readings:
 *   ORC_TAIL_VISIBLE (the library's default): it is eligible and its key is
 *       the rounded mean of its rows at positions <= t;
 *   ORC_TAIL_EXCLUDE: it is not eligible (its tokens are still in the sliding
 *       window, whose length is at least B);
 *   ORC_TAIL_WHOLE: it is eligible and its key averages all of its rows that
 *       exist in k_seq (positions < T), including positions after t.
 * Complete blocks are the same under every reading, and in every reading a
 * candidate token is a position <= t. */
enum { ORC_TAIL_VISIBLE = 0, ORC_TAIL_EXCLUDE = 1, ORC_TAIL_WHOLE = 2 };

int orc_select_one(const int8_t *q_idx, const int8_t *k_seq, int T, int t,
                   int d, int B, int P, int K, int tail,
                   int32_t *blk_ids, int32_t *blk_cnt, int32_t *topk, int32_t *topk_cnt)
{
    if (t < 0 || t >= T || d <= 0 || B <= 0 || P <= 0 || K < 0) return -1;
    if (tail < ORC_TAIL_VISIBLE || tail > ORC_TAIL_WHOLE) return -1;
    /* eligible blocks: those with a visible token (j*B <= t), or only the
     * complete ones ((j+1)*B <= t+1) when the partial block is excluded */
    int n_elig = (tail == ORC_TAIL_EXCLUDE) ? (t + 1) / B : t / B + 1;
    /* last row a block key may average: t, or the last row of the cache */
    int key_limit = (tail == ORC_TAIL_WHOLE) ? T - 1 : t;

    /* block scores */
    scored *blocks = malloc(sizeof(scored) * (size_t)(n_elig > 0 ? n_elig : 1));
    int8_t *key = malloc((size_t)d);
    if (!blocks || !key) { free(blocks); free(key); return -1; }
    for (int j = 0; j < n_elig; j++) {
        orc_block_key(k_seq, d, B, j, key_limit, key);
        blocks[j].score = dot_i8(q_idx, key, d);
        blocks[j].id = j;
    }
    int n_pool = n_elig;
    if (n_elig > P) {
        qsort(blocks, (size_t)n_elig, sizeof(scored), by_score_then_id);
        n_pool = P;
    }
    int32_t *pool = malloc(sizeof(int32_t) * (size_t)(n_pool > 0 ? n_pool : 1));
    if (!pool) { free(key); free(blocks); return -1; }
    for (int i = 0; i < n_pool; i++) pool[i] = blocks[i].id;
    qsort(pool, (size_t)n_pool, sizeof(int32_t), by_id);
    for (int i = 0; i < P; i++) blk_ids[i] = (i < n_pool) ? pool[i] : -1;
    *blk_cnt = n_pool;

    int bad = orc_topk_one(q_idx, k_seq, T, t, d, B, pool, n_pool, K, topk, topk_cnt);
    free(pool); free(key); free(blocks);
    return bad;
}

/* Queries [q_begin, q_end) of a batch.  q_idx [n_q][d]; k_idx [S][T][d];
 * blk_ids [n_q][P]; topk [n_q][K].  q_pos holds token positions; with ratio
 * r the query selects over its visible main-KV entries (T of them stored per
 * sequence), its last visible entry taking the place of t above, and a query
 * that sees no entry selects nothing.  Returns the number of failed queries. */
int orc_select_batch(int q_begin, int q_end, const int8_t *q_idx,
                     const int32_t *q_seq, const int32_t *q_pos,
                     const int8_t *k_idx, int S, int T, int d, int B, int P, int K, int tail,
                     int ratio, int32_t *blk_ids, int32_t *blk_cnt, int32_t *topk, int32_t *topk_cnt)
{
    int bad = 0;
    for (int i = q_begin; i < q_end; i++) {
        int s = q_seq[i];
        if (s < 0 || s >= S) { bad++; continue; }
        const int n_vis = orc_visible_entries(q_pos[i], ratio);
        if (n_vis < 0) { bad++; continue; }
        if (n_vis == 0) {
            empty_selection(blk_ids + (size_t)i * P, P, blk_cnt + i);
            empty_selection(topk + (size_t)i * K, K, topk_cnt + i);
            continue;
        }
        bad += orc_select_one(q_idx + (size_t)i * d, k_idx + (size_t)s * T * d, T, n_vis - 1,
                              d, B, P, K, tail, blk_ids + (size_t)i * P, blk_cnt + i,
                              topk + (size_t)i * K, topk_cnt + i) != 0;
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Steps 6-7: window and attention for one query and one layer.             */
/* ------------------------------------------------------------------------ */

/* One softmax per head over the concatenation of
 *   - the selected main-KV entries p in topk[0..cnt) (shared main K/V rows), and
 *   - the window positions max(0, t-W+1) .. t (this layer's own window K/V,
 *     where row r of k_swa/v_swa holds position swa_first + r),
 * with logits scale * <Q[h], K[p]>.  Entries at the same position in both sets
 * are different vectors and both count.
 *   q     : [H][D] of this query and layer
 *   k_main, v_main : one sequence's main K/V [T][D]
 *   k_swa, v_swa   : one sequence's window K/V [swa_len][D]
 *   out   : [H][D] fp64, lse: [H] fp64 (natural log of the softmax normaliser)
 * Returns 0, or -1 when the window rows do not cover the window or the set is
 * empty. */
int orc_attend_one(const void *q, const void *k_main, const void *v_main, int T,
                   const void *k_swa, const void *v_swa, int swa_first, int swa_len,
                   const int32_t *topk, int cnt, int t, int W, int H, int D, int elem,
                   double scale, double *out, double *lse)
{
    int w0 = t - W + 1;
    if (w0 < 0) w0 = 0;
    int nw = (W > 0) ? t - w0 + 1 : 0;
    if (nw > 0 && (w0 < swa_first || t >= swa_first + swa_len)) return -1;
    if (cnt + nw <= 0) return -1;
    double *logit = malloc(sizeof(double) * (size_t)(cnt + nw));
    if (!logit) return -1;

    for (int h = 0; h < H; h++) {
        /* logits */
        for (int i = 0; i < cnt; i++) {
            int p = topk[i];
            if (p < 0 || p >= T) { free(logit); return -1; }
            double acc = 0.0;
            for (int c = 0; c < D; c++)
                acc += load_elem(q, elem, (size_t)h * D + c) *
                       load_elem(k_main, elem, (size_t)p * D + c);
            logit[i] = scale * acc;
        }
        for (int i = 0; i < nw; i++) {
            int r = w0 + i - swa_first;
            double acc = 0.0;
            for (int c = 0; c < D; c++)
                acc += load_elem(q, elem, (size_t)h * D + c) *
                       load_elem(k_swa, elem, (size_t)r * D + c);
            logit[cnt + i] = scale * acc;
        }
        /* softmax normaliser */
        double m = -INFINITY;
        for (int i = 0; i < cnt + nw; i++)
            if (logit[i] > m) m = logit[i];
        double z = 0.0;
        for (int i = 0; i < cnt + nw; i++) {
            logit[i] = exp(logit[i] - m);    /* now the unnormalised weight */
            z += logit[i];
        }
        /* weighted sum of values */
        for (int c = 0; c < D; c++) {
            double acc = 0.0;
            for (int i = 0; i < cnt; i++)
                acc += logit[i] * load_elem(v_main, elem, (size_t)topk[i] * D + c);
            for (int i = 0; i < nw; i++)
                acc += logit[cnt + i] *
                       load_elem(v_swa, elem, (size_t)(w0 + i - swa_first) * D + c);
            out[(size_t)h * D + c] = acc / z;
        }
        lse[h] = m + log(z);
    }
    free(logit);
    return 0;
}

/* Queries [q_begin, q_end) of one layer.
 *   q [n_q][H][D]; k_main/v_main [S][T][D]; k_swa/v_swa [S][swa_len][D];
 *   topk [n_q][K_stride] with topk_cnt [n_q] (cnt may be 0: window only);
 *   out [n_q][H][D] fp64; lse [n_q][H] fp64.
 * Returns the number of failed queries. */
int orc_attend_batch(int q_begin, int q_end, const void *q,
                     const int32_t *q_seq, const int32_t *q_pos,
                     const void *k_main, const void *v_main, int S, int T,
                     const void *k_swa, const void *v_swa, int swa_first, int swa_len,
                     const int32_t *topk, const int32_t *topk_cnt, int K_stride,
                     int W, int H, int D, int elem, double scale, double *out, double *lse)
{
    size_t esz = (elem == ORC_F32) ? 4 : 2;
    int bad = 0;
    for (int i = q_begin; i < q_end; i++) {
        int s = q_seq[i];
        if (s < 0 || s >= S) { bad++; continue; }
        const char *qb = (const char *)q + (size_t)i * H * D * esz;
        const char *km = (const char *)k_main + (size_t)s * T * D * esz;
        const char *vm = (const char *)v_main + (size_t)s * T * D * esz;
        const char *ks = (const char *)k_swa + (size_t)s * swa_len * D * esz;
        const char *vs = (const char *)v_swa + (size_t)s * swa_len * D * esz;
        int cnt = topk ? topk_cnt[i] : 0;
        bad += orc_attend_one(qb, km, vm, T, ks, vs, swa_first, swa_len,
                              topk ? topk + (size_t)i * K_stride : NULL, cnt, q_pos[i], W,
                              H, D, elem, scale, out + (size_t)i * H * D, lse + (size_t)i * H) != 0;
    }
    return bad;
}
