/*
 * qsa_oracle.c -- plain fp64 CPU oracle for route-sparse GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * It is the plain definition, written for a reader to check by eye, with no
 * blocking, fusion or reordering:
 *
 *  - Route set of a query row (flex_qsa page, `_routes_to_membership`
 *    parameters and module description; fa4_qsa page, `_preprocess`
 *    parameters; qsa page, `qsa_gqa_attention` parameters): every slot value
 *    x is widened to int64; x is a valid key iff 0 <= x < kv_length (negative
 *    IDs, -1 padding and out-of-range values, including huge int64 values,
 *    are ignored); a repeated ID counts once.  R(b,i) is that set in
 *    ascending order.
 *  - Membership table (fa4_qsa page, `_preprocess` return value): uint8
 *    [B, S_q, ldm], 1 iff column c is in R(b,i); columns past kv_length are
 *    the row padding and hold 0.
 *  - Tile classes (fa4_qsa page, `_block_kinds` and `_compact_blocks`):
 *    int32 [B, ceil(S_q/128), ceil(kv_length/128)]; 0 when no member pair
 *    lies in the tile, 2 when every in-range pair of the tile is a member,
 *    1 otherwise.
 *  - Attention (flex_qsa page, module description and
 *    `flex_sparse_gqa_attention`; fa4_qsa page, `fa4_sparse_gqa_attention`;
 *    qsa page, `_gathered_qsa_gqa_attention_chunk` grouped layout): query
 *    head h reads KV head h / (Hq/Hkv); over j in R(b,i),
 *    s_j = scale * <q[b,i,h,:], k[b,j,hk,:]>, o = sum_j softmax(s)_j v[b,j,hk,:];
 *    an empty R gives exactly zero; no causal or other mask is added.
 *    All arithmetic is fp64 on the exact bfloat16 input values.
 *  - Block lists of a tile-class table (fa4_qsa page, `_compact_blocks` and
 *    `_preprocess`): per block row (forward) and per block column (reverse),
 *    the count and ascending indices of partial and of full tiles, see
 *    `oracle_tile_lists`.
 *  - Route selection (qsa page, `select_qsa_token_ids`): per query row the
 *    best compressed blocks by sum over index heads of relu(q . k) / sqrt(D),
 *    expanded to token IDs, plus the incomplete causal tail, see
 *    `oracle_select_token_ids`.
 *  - Log-sum-exp of each row's scaled scores and the first-order gradients
 *    dq, dk, dv of that attention (fa4_qsa page: FA4 owns first-order
 *    autograd; empty rows have zero output and zero gradients): the softmax
 *    Jacobian written out per (row, head), see `oracle_backward`.
 *
 * Rows are independent, so each entry point runs its outer row loop under
 * OpenMP; that changes no per-row arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int cmp_int64(const void *a, const void *b) {
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* R(row): ascending distinct valid IDs of one row of K slots; returns |R|. */
static int64_t route_set(const int64_t *slots, int64_t K, int64_t kv_length, int64_t *out) {
    int64_t n = 0;
    for (int64_t s = 0; s < K; ++s) {
        int64_t x = slots[s];
        if (x >= 0 && x < kv_length) out[n++] = x;
    }
    qsort(out, (size_t)n, sizeof(int64_t), cmp_int64);
    int64_t m = 0;
    for (int64_t j = 0; j < n; ++j)
        if (m == 0 || out[j] != out[m - 1]) out[m++] = out[j];
    return m;
}

static double bf16_to_double(uint16_t h) {
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* route_list [rows, K] int32 (R ascending, then -1) and route_count [rows]. */
void oracle_route_lists(const int64_t *routes, int64_t rows, int64_t K, int64_t kv_length,
                        int32_t *route_list, int32_t *route_count) {
#pragma omp parallel
    {
        int64_t *set = (int64_t *)malloc((size_t)K * sizeof(int64_t));
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t n = route_set(routes + r * K, K, kv_length, set);
            for (int64_t j = 0; j < K; ++j) route_list[r * K + j] = j < n ? (int32_t)set[j] : -1;
            route_count[r] = (int32_t)n;
        }
        free(set);
    }
}

/* membership [rows, ldm] uint8: 1 iff the column is in the row's route set. */
void oracle_membership(const int64_t *routes, int64_t rows, int64_t K, int64_t kv_length, int64_t ldm,
                       uint8_t *membership) {
#pragma omp parallel
    {
        int64_t *set = (int64_t *)malloc((size_t)K * sizeof(int64_t));
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < rows; ++r) {
            uint8_t *row = membership + r * ldm; /* int64 offset throughout */
            for (int64_t c = 0; c < ldm; ++c) row[c] = 0;
            int64_t n = route_set(routes + r * K, K, kv_length, set);
            for (int64_t j = 0; j < n; ++j) row[set[j]] = 1;
        }
        free(set);
    }
}

/* tile_class [B, ceil(S_q/128), ceil(kv_length/128)] int32 in {0, 1, 2}. */
void oracle_tile_class(const int64_t *routes, int64_t B, int64_t S_q, int64_t K, int64_t kv_length,
                       int32_t *tile_class) {
    const int64_t T = 128;
    const int64_t n_ti = (S_q + T - 1) / T, n_tj = (kv_length + T - 1) / T;
#pragma omp parallel
    {
        int64_t *set = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        int64_t *members = (int64_t *)malloc((size_t)n_tj * sizeof(int64_t));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t ti = 0; ti < n_ti; ++ti) {
                int64_t r0 = ti * T, r1 = r0 + T < S_q ? r0 + T : S_q;
                for (int64_t tj = 0; tj < n_tj; ++tj) members[tj] = 0;
                for (int64_t i = r0; i < r1; ++i) {
                    int64_t n = route_set(routes + (b * S_q + i) * K, K, kv_length, set);
                    for (int64_t j = 0; j < n; ++j) members[set[j] / T] += 1;
                }
                for (int64_t tj = 0; tj < n_tj; ++tj) {
                    int64_t c0 = tj * T, c1 = c0 + T < kv_length ? c0 + T : kv_length;
                    int64_t pairs = (r1 - r0) * (c1 - c0);
                    int32_t cls = members[tj] == 0 ? 0 : (members[tj] == pairs ? 2 : 1);
                    tile_class[(b * n_ti + ti) * n_tj + tj] = cls;
                }
            }
        }
        free(set);
        free(members);
    }
}

/*
 * out [B, row_end - row_begin, Hq, D] fp64: attention of query rows
 * [row_begin, row_end) of every batch row.  q is [B,S_q,Hq,D], k and v are
 * [B,S_kv,Hkv,D], all contiguous bfloat16 bit patterns; routes [B,S_q,K].
 */
void oracle_forward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *routes,
                    int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K,
                    double scale, int64_t row_begin, int64_t row_end, double *out) {
    const int64_t G = Hq / Hkv;
    const int64_t n_rows = row_end - row_begin;
#pragma omp parallel
    {
        int64_t *set = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        double *score = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 4) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t i = row_begin; i < row_end; ++i) {
                int64_t n = route_set(routes + (b * S_q + i) * K, K, S_kv, set);
                for (int64_t h = 0; h < Hq; ++h) {
                    int64_t hk = h / G;
                    const uint16_t *qv = q + ((b * S_q + i) * Hq + h) * D;
                    double *o = out + ((b * n_rows + (i - row_begin)) * Hq + h) * D;
                    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                    if (n == 0) continue; /* empty route set: exactly zero */
                    double m = -INFINITY;
                    for (int64_t j = 0; j < n; ++j) {
                        const uint16_t *kv = k + ((b * S_kv + set[j]) * Hkv + hk) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qv[d]) * bf16_to_double(kv[d]);
                        score[j] = scale * dot;
                        if (score[j] > m) m = score[j];
                    }
                    double denom = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        double w = exp(score[j] - m);
                        denom += w;
                        const uint16_t *vv = v + ((b * S_kv + set[j]) * Hkv + hk) * D;
                        for (int64_t d = 0; d < D; ++d) o[d] += w * bf16_to_double(vv[d]);
                    }
                    for (int64_t d = 0; d < D; ++d) o[d] /= denom;
                }
            }
        }
        free(set);
        free(score);
    }
}

/*
 * lse [B, row_end - row_begin, Hq] fp64: natural-log log-sum-exp of the
 * scaled scores of each (query row, head), log sum_j exp(s_j) over j in
 * R(b,i); -inf for an empty route set.  This is the per-row statistic a
 * forward pass keeps for its backward (fa4_qsa page: the FA4 kernel owns
 * first-order autograd).
 */
void oracle_lse(const uint16_t *q, const uint16_t *k, const int64_t *routes, int64_t B, int64_t S_q,
                int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K, double scale, int64_t row_begin,
                int64_t row_end, double *lse) {
    const int64_t G = Hq / Hkv;
    const int64_t n_rows = row_end - row_begin;
#pragma omp parallel
    {
        int64_t *set = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        double *score = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 4) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t i = row_begin; i < row_end; ++i) {
                int64_t n = route_set(routes + (b * S_q + i) * K, K, S_kv, set);
                for (int64_t h = 0; h < Hq; ++h) {
                    int64_t hk = h / G;
                    const uint16_t *qv = q + ((b * S_q + i) * Hq + h) * D;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < n; ++j) {
                        const uint16_t *kv = k + ((b * S_kv + set[j]) * Hkv + hk) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qv[d]) * bf16_to_double(kv[d]);
                        score[j] = scale * dot;
                        if (score[j] > m) m = score[j];
                    }
                    double sum = 0.0;
                    for (int64_t j = 0; j < n; ++j) sum += exp(score[j] - m);
                    lse[(b * n_rows + (i - row_begin)) * Hq + h] = n == 0 ? -INFINITY : m + log(sum);
                }
            }
        }
        free(set);
        free(score);
    }
}

/*
 * Gradients of the attention above for an upstream gradient dout
 * [B,S_q,Hq,D] (bfloat16 bits), i.e. of L = sum dout * out (fa4_qsa page:
 * first-order autograd; flex_qsa page, module description, and fa4_qsa
 * page, `fa4_sparse_gqa_attention`: rows whose routes are all invalid have
 * zero output and zero gradients).  For a (b, i, h) with non-empty R:
 *
 *   p_j   = softmax(s)_j                       (s_j as in the forward)
 *   dp_j  = <dout[b,i,h,:], v[b,j,hk,:]>
 *   ds_j  = p_j * (dp_j - sum_l p_l dp_l)      (softmax Jacobian)
 *   dq[b,i,h,:]   = scale * sum_j ds_j k[b,j,hk,:]
 *   dk[b,j,hk,:] += scale * ds_j q[b,i,h,:]     over every (i, h) routing j
 *   dv[b,j,hk,:] += p_j dout[b,i,h,:]           over every (i, h) routing j
 *
 * dq is produced for query rows [row_begin, row_end) as [B, rows, Hq, D];
 * dk and dv for keys [key_begin, key_end) as [B, keys, Hkv, D], summed over
 * all query rows.  Keys that no row routes get zero.  Rows run in parallel;
 * the dk/dv sums use atomic adds (fp64, so the summation order does not
 * matter at the tolerances used).
 */
void oracle_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *dout,
                     const int64_t *routes, int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                     int64_t D, int64_t K, double scale, int64_t row_begin, int64_t row_end, int64_t key_begin,
                     int64_t key_end, double *dq, double *dk, double *dv) {
    const int64_t G = Hq / Hkv;
    const int64_t n_rows = row_end - row_begin, n_keys = key_end - key_begin;
    for (int64_t x = 0; x < B * n_rows * Hq * D; ++x) dq[x] = 0.0;
    for (int64_t x = 0; x < B * n_keys * Hkv * D; ++x) dk[x] = dv[x] = 0.0;
#pragma omp parallel
    {
        int64_t *set = (int64_t *)malloc((size_t)K * sizeof(int64_t));
        double *p = (double *)malloc((size_t)K * sizeof(double));
        double *dp = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 4) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t i = 0; i < S_q; ++i) {
                int64_t n = route_set(routes + (b * S_q + i) * K, K, S_kv, set);
                int want_dq = i >= row_begin && i < row_end;
                int touches = 0;
                for (int64_t j = 0; j < n; ++j) touches |= set[j] >= key_begin && set[j] < key_end;
                if (n == 0 || (!want_dq && !touches)) continue; /* empty rows: zero gradients */
                for (int64_t h = 0; h < Hq; ++h) {
                    int64_t hk = h / G;
                    const uint16_t *qv = q + ((b * S_q + i) * Hq + h) * D;
                    const uint16_t *gv = dout + ((b * S_q + i) * Hq + h) * D;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < n; ++j) {
                        const uint16_t *kv = k + ((b * S_kv + set[j]) * Hkv + hk) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qv[d]) * bf16_to_double(kv[d]);
                        p[j] = scale * dot;
                        if (p[j] > m) m = p[j];
                    }
                    double denom = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        p[j] = exp(p[j] - m);
                        denom += p[j];
                    }
                    double pdp = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        p[j] /= denom;
                        const uint16_t *vv = v + ((b * S_kv + set[j]) * Hkv + hk) * D;
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(gv[d]) * bf16_to_double(vv[d]);
                        dp[j] = dot;
                        pdp += p[j] * dp[j];
                    }
                    for (int64_t j = 0; j < n; ++j) {
                        double ds = p[j] * (dp[j] - pdp);
                        const uint16_t *kv = k + ((b * S_kv + set[j]) * Hkv + hk) * D;
                        if (want_dq) {
                            double *o = dq + ((b * n_rows + (i - row_begin)) * Hq + h) * D;
                            for (int64_t d = 0; d < D; ++d) o[d] += scale * ds * bf16_to_double(kv[d]);
                        }
                        if (set[j] >= key_begin && set[j] < key_end) {
                            double *gk = dk + ((b * n_keys + (set[j] - key_begin)) * Hkv + hk) * D;
                            double *gw = dv + ((b * n_keys + (set[j] - key_begin)) * Hkv + hk) * D;
                            for (int64_t d = 0; d < D; ++d) {
#pragma omp atomic
                                gk[d] += scale * ds * bf16_to_double(qv[d]);
#pragma omp atomic
                                gw[d] += p[j] * bf16_to_double(gv[d]);
                            }
                        }
                    }
                }
            }
        }
        free(set);
        free(p);
        free(dp);
    }
}

/*
 * Block lists of a tile-class table (fa4_qsa page, `_compact_blocks`: partial
 * and full block columns of each block row, int32 counts [batch, 1, rows];
 * `_preprocess`: forward and reverse block lists).  kinds is int32
 * [B, n_rows, n_cols] with 0 absent, 1 partial, 2 full.
 *
 * Forward, per (b, row) and per kind k in {1, 2}:
 *   count[b][row]    = number of columns whose class is k;
 *   idx[b][row][:]   = those columns in ascending order, followed by every
 *                      other column in ascending order (each index row is a
 *                      permutation of 0 .. n_cols - 1; only the first count
 *                      entries are meaningful).
 * Reverse, per (b, col): the same over rows of that column.
 * Any output pointer may be NULL (that list is not produced).
 */
static void compact_line(const int32_t *kinds, int64_t n, int64_t stride, int32_t want, int32_t *count,
                         int32_t *idx) {
    int64_t m = 0;
    for (int64_t x = 0; x < n; ++x)
        if (kinds[x * stride] == want) {
            if (idx) idx[m] = (int32_t)x;
            ++m;
        }
    if (count) *count = (int32_t)m;
    if (idx) {
        int64_t r = m;
        for (int64_t x = 0; x < n; ++x)
            if (kinds[x * stride] != want) idx[r++] = (int32_t)x;
    }
}

void oracle_tile_lists(const int32_t *kinds, int64_t B, int64_t n_rows, int64_t n_cols, int32_t *partial_count,
                       int32_t *partial_idx, int32_t *full_count, int32_t *full_idx, int32_t *rev_partial_count,
                       int32_t *rev_partial_idx, int32_t *rev_full_count, int32_t *rev_full_idx) {
    for (int64_t b = 0; b < B; ++b) {
        const int32_t *kb = kinds + b * n_rows * n_cols;
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t o = b * n_rows + r;
            compact_line(kb + r * n_cols, n_cols, 1, 1, partial_count ? partial_count + o : NULL,
                         partial_idx ? partial_idx + o * n_cols : NULL);
            compact_line(kb + r * n_cols, n_cols, 1, 2, full_count ? full_count + o : NULL,
                         full_idx ? full_idx + o * n_cols : NULL);
        }
        for (int64_t c = 0; c < n_cols; ++c) {
            const int64_t o = b * n_cols + c;
            compact_line(kb + c, n_rows, n_cols, 1, rev_partial_count ? rev_partial_count + o : NULL,
                         rev_partial_idx ? rev_partial_idx + o * n_rows : NULL);
            compact_line(kb + c, n_rows, n_cols, 2, rev_full_count ? rev_full_count + o : NULL,
                         rev_full_idx ? rev_full_idx + o * n_rows : NULL);
        }
    }
}

/*
 * Route selection by compressed-block scores (qsa page,
 * `select_qsa_token_ids`; the page's indexer class for the output
 * width).
 *
 * Inputs: index queries iq [B, S_q, H, D] and compressed block keys
 * ck [B, n_blocks, D] (one key head), contiguous bfloat16 bit patterns;
 * seq_lens [B] right-padded logical lengths in global positions.  Local
 * query row i stands at global position t = q_offset + i.  With
 * c = compress_ratio, kb = token_budget / c (integer division) and
 * W = token_budget + c - 1 slots per row:
 *
 *   - a row with t >= seq_lens[b] is a padding query: every slot is -1;
 *   - otherwise nv = floor((t + 1) / c) complete blocks are visible, and
 *     block j scores  s_j = sum_h max(0, <iq[b,i,h,:], ck[b,j,:]>) / sqrt(D);
 *   - the m = min(kb, nv) best blocks are kept, best meaning the larger
 *     score and, between equal scores, the smaller block index;
 *   - slots [0, m*c) hold the kept blocks in ascending block order, each
 *     expanded to its c token IDs j*c .. j*c + c - 1; slots [m*c, token_budget)
 *     are -1;
 *   - slots [token_budget, token_budget + (t + 1) - nv*c) hold the tokens of
 *     the incomplete causal tail, nv*c .. t; the remaining slots are -1.
 *
 * Scores are fp64 on the exact bfloat16 values; the order of the kept
 * blocks, the tie rule and the fixed slot layout are readings of the page
 * (it orders none of them).  out is [B, row_end - row_begin, W] int32.
 */
typedef struct {
    double score;
    int64_t block;
} scored_block;

static int cmp_best_first(const void *a, const void *b) {
    const scored_block *x = (const scored_block *)a, *y = (const scored_block *)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    return (x->block > y->block) - (x->block < y->block);
}

/* s_j of one query row against one block key, fp64. */
static double block_score(const uint16_t *qrow, const uint16_t *key, int64_t H, int64_t D) {
    double total = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += bf16_to_double(qrow[h * D + d]) * bf16_to_double(key[d]);
        total += dot > 0.0 ? dot : 0.0;
    }
    return total / sqrt((double)D);
}

/* scores [B, row_end - row_begin, n_blocks] fp64: s_j for every block, visible or not. */
void oracle_block_scores(const uint16_t *iq, const uint16_t *ck, int64_t B, int64_t S_q, int64_t H, int64_t D,
                         int64_t n_blocks, int64_t row_begin, int64_t row_end, double *scores) {
    const int64_t n_rows = row_end - row_begin;
#pragma omp parallel for schedule(dynamic, 4) collapse(2)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = row_begin; i < row_end; ++i)
            for (int64_t j = 0; j < n_blocks; ++j)
                scores[(b * n_rows + (i - row_begin)) * n_blocks + j] =
                    block_score(iq + (b * S_q + i) * H * D, ck + (b * n_blocks + j) * D, H, D);
}

void oracle_select_token_ids(const uint16_t *iq, const uint16_t *ck, const int64_t *seq_lens, int64_t B,
                             int64_t S_q, int64_t H, int64_t D, int64_t n_blocks, int64_t q_offset,
                             int64_t token_budget, int64_t compress_ratio, int64_t row_begin, int64_t row_end,
                             int32_t *out) {
    const int64_t c = compress_ratio;
    const int64_t kb = token_budget / c;
    const int64_t W = token_budget + c - 1;
    const int64_t n_rows = row_end - row_begin;
#pragma omp parallel
    {
        scored_block *cand = (scored_block *)malloc((size_t)(n_blocks > 0 ? n_blocks : 1) * sizeof(scored_block));
        int64_t *kept = (int64_t *)malloc((size_t)(n_blocks > 0 ? n_blocks : 1) * sizeof(int64_t));
#pragma omp for schedule(dynamic, 4) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t i = row_begin; i < row_end; ++i) {
                int32_t *o = out + (b * n_rows + (i - row_begin)) * W;
                for (int64_t s = 0; s < W; ++s) o[s] = -1;
                const int64_t t = q_offset + i;
                if (t >= seq_lens[b]) continue; /* padding query */
                const int64_t nv = (t + 1) / c; /* <= n_blocks: the caller checks it */
                for (int64_t j = 0; j < nv; ++j) {
                    cand[j].score = block_score(iq + (b * S_q + i) * H * D, ck + (b * n_blocks + j) * D, H, D);
                    cand[j].block = j;
                }
                qsort(cand, (size_t)nv, sizeof(scored_block), cmp_best_first);
                const int64_t m = kb < nv ? kb : nv;
                for (int64_t r = 0; r < m; ++r) kept[r] = cand[r].block;
                qsort(kept, (size_t)m, sizeof(int64_t), cmp_int64);
                for (int64_t r = 0; r < m; ++r)
                    for (int64_t u = 0; u < c; ++u) o[r * c + u] = (int32_t)(kept[r] * c + u);
                for (int64_t u = 0; nv * c + u <= t; ++u) o[token_budget + u] = (int32_t)(nv * c + u);
            }
        }
        free(cand);
        free(kept);
    }
}
