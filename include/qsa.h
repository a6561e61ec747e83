/*
 * qsa.h -- C ABI of libqsa: route-sparse grouped-query attention (forward
 * and first-order backward) on AMD Instinct MI355X (gfx950).
 *
 * Every query row attends exactly to its own set of key/value token IDs
 * ("routes").  The operation is the one defined on the route-sparse GQA
 * pages:
 *   - flex_qsa page, module description: padded batches, packed THD rows and
 *     context parallelism all reduce to "each query row attends to its route
 *     IDs"; rows without a valid route give exactly zero output.
 *   - fa4_qsa page, `_preprocess` and `fa4_sparse_gqa_attention`: a
 *     repeated ID selects its token once; an ID outside [0, kv_length),
 *     however large, is ignored; no causal or other mask is added beyond
 *     the routes.
 *   - qsa page, `_gathered_qsa_gqa_attention_chunk`: grouped query layout
 *     [B, Q, Hkv, G, D], i.e. query head h reads KV head h / G, G = Hq / Hkv.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing, frees nothing and keeps no pointer or other
 *     state after a call returns; it is safe to call from several threads.
 *   - Sizes and strides are int64_t; strides are in ELEMENTS.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it; no call synchronises the host or reads device memory
 *     on the host.
 *   - Every output byte is written by the library (list padding, membership
 *     row padding, zero rows): callers need not clear anything.
 *   - Return value: QSA_OK (0) or a negative QSA_ERR_* status.  Argument
 *     checks are host-only; when one fails nothing is enqueued.  Route
 *     VALUES are data, never errors: invalid IDs are ignored.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define QSA_OK 0
#define QSA_ERR_NULL_POINTER -1 /* a required pointer is NULL                          */
#define QSA_ERR_EMPTY_DIM -2    /* B, S_q, S_kv, Hq, Hkv, D or K < 1 (pages: nonempty)  */
#define QSA_ERR_KV_LENGTH -3    /* kv_length < 1 or > 2^31 (IDs are stored as int32)   */
#define QSA_ERR_HEADS -4        /* Hq is not a positive multiple of Hkv                */
#define QSA_ERR_HEAD_DIM -5     /* D not in {64, 128, 256}                             */
#define QSA_ERR_ROUTE_DTYPE -6  /* routes_dtype is neither QSA_INT32 nor QSA_INT64     */
#define QSA_ERR_SCALE -7        /* scale is not finite and > 0                         */
#define QSA_ERR_LAYOUT -8       /* last stride != 1, or a row/pointer not 16-B aligned */
#define QSA_ERR_ALIAS -9        /* an output overlaps an input or another output       */
#define QSA_ERR_WORKSPACE -10   /* workspace NULL or smaller than required             */
#define QSA_ERR_LIMIT -11       /* a size beyond a library limit: K > QSA_MAX_ROUTES,  */
                                /* G > QSA_MAX_GROUP, B*S_q >= 2^24, more index heads, */
                                /* kept or visible blocks than the selection limits,   */
                                /* a launch of 2^32 or more work-items (one grid       */
                                /* dimension holds fewer), or strides whose element    */
                                /* offsets overflow 64 bits                            */
#define QSA_ERR_HIP -12         /* a HIP launch reported an error                      */
#define QSA_ERR_SELECTION -13   /* token_budget or compress_ratio < 1, or query rows   */
                                /* outside [0, S_global) (route selection)             */
#define QSA_ERR_SCRATCH_LIMIT -14 /* qsa_forward_noalloc: the call needs more than its  */
                                  /* fixed scratch (QSA_NOALLOC_SCRATCH_BYTES)          */

/* ---- constants --------------------------------------------------------- */
#define QSA_INT32 0          /* routes are int32_t (sign-extended before the checks) */
#define QSA_INT64 1          /* routes are int64_t                                    */
#define QSA_TILE 128         /* rows and columns of one membership tile              */
#define QSA_MAX_ROUTES 16384 /* largest K (route slots per query row)               */
#define QSA_MAX_GROUP 16     /* largest G = Hq / Hkv                                */
#define QSA_MAX_SELECT_BLOCKS 4096   /* largest token_budget / compress_ratio          */
#define QSA_MAX_VISIBLE_BLOCKS 65536 /* largest floor(S_global / compress_ratio)       */
#define QSA_MAX_INDEX_HEADS 64       /* largest H (index heads) of route selection     */
#define QSA_NOALLOC_SCRATCH_BYTES (64u << 20) /* device scratch of qsa_forward_noalloc (64 MiB) */

/*
 * qsa_preprocess -- validate, deduplicate and compact the routes; optionally
 * build the uint8 membership table and the 128x128 tile classes.
 *
 * Definition (fa4_qsa page, `_preprocess`, `_block_kinds`; flex_qsa page,
 * `_routes_to_membership` and `_membership_flat_offset`): a slot value x
 * (int32 values sign-extended to int64) is a valid key iff
 * 0 <= x < kv_length; R(b,i) = the ascending set of distinct valid values of
 * row (b,i).
 *
 *   routes        [B, S_q, K] int32 or int64 (`routes_dtype`), any strides
 *                 (`route_strides`, elements, may be 0 or negative).
 *   kv_length     number of physical K/V rows, 1 <= kv_length <= 2^31.
 *   route_list    OUT [B, S_q, K] int32, contiguous: R(b,i) ascending, then
 *                 -1 in the remaining K - |R| slots.
 *   route_count   OUT [B, S_q] int32, contiguous: |R(b,i)|.
 *   membership    OUT, nullable: [B, S_q, ldm] uint8, contiguous,
 *                 ldm = round_up(kv_length, 128); 1 iff the column is in
 *                 R(b,i), 0 elsewhere (padding columns included).  Offsets
 *                 are 64-bit: the table may exceed 2^31 bytes.
 *   tile_class    OUT, nullable: [B, ceil(S_q/128), ceil(kv_length/128)]
 *                 int32, contiguous: 0 = no member pair in the tile,
 *                 2 = every in-range pair of the tile is a member,
 *                 1 = otherwise.  Independent of `membership`.
 *
 * Errors: NULL_POINTER, EMPTY_DIM, KV_LENGTH, ROUTE_DTYPE, LIMIT (K),
 * LAYOUT (route_count/list not 4-B aligned, membership not 16-B aligned),
 * ALIAS (outputs overlap each other or `routes`), HIP.
 */
int qsa_preprocess(const void *routes, int routes_dtype, int64_t B, int64_t S_q, int64_t K,
                   const int64_t route_strides[3], int64_t kv_length, int32_t *route_list,
                   int32_t *route_count, uint8_t *membership, int32_t *tile_class, void *stream);

/*
 * qsa_tile_lists -- forward and reverse partial/full block lists of a
 * tile-class table (the block-sparse format of FlexAttention's BlockMask and
 * the pages' FA4 path).
 *
 * Definition (fa4_qsa page, `_compact_blocks`: partial and full block
 * columns of each block row, int32 counts [batch, 1, block_rows];
 * `_preprocess`: forward and reverse block lists).  For each line -- a block
 * row for the forward lists, a block column for the reverse ones -- and each
 * kind (1 partial, 2 full): the number of tiles of that kind, and an index
 * row with their positions in ascending order followed by every other
 * position in ascending order (a permutation; only the first count entries
 * are meaningful).
 *
 *   tile_class        [B, n_rows, n_cols] int32 (0/1/2), contiguous, as
 *                     qsa_preprocess writes it.  Other values count as
 *                     neither kind.
 *   partial_count     OUT, nullable: [B, 1, n_rows] int32
 *   partial_idx       OUT, nullable: [B, 1, n_rows, n_cols] int32
 *   full_count, full_idx                 OUT, nullable: same shapes, full tiles
 *   rev_partial_count OUT, nullable: [B, 1, n_cols] int32
 *   rev_partial_idx   OUT, nullable: [B, 1, n_cols, n_rows] int32
 *   rev_full_count, rev_full_idx         OUT, nullable: same shapes, full tiles
 * All contiguous, 4-B aligned, not overlapping each other or tile_class.
 * Errors: NULL_POINTER (tile_class), EMPTY_DIM, LAYOUT, ALIAS, LIMIT, HIP.
 */
int qsa_tile_lists(const int32_t *tile_class, int64_t B, int64_t n_rows, int64_t n_cols, int32_t *partial_count,
                   int32_t *partial_idx, int32_t *full_count, int32_t *full_idx, int32_t *rev_partial_count,
                   int32_t *rev_partial_idx, int32_t *rev_full_count, int32_t *rev_full_idx, void *stream);

/*
 * qsa_attention_workspace_size -- recommended bytes of device workspace for
 * the attention kernels (qsa_forward_preprocessed), 0 when these shapes need
 * none.
 *
 * When one KV head's K and V rows span more than 16 MiB (S_kv * 4 * D
 * bytes, four times one XCD's L2), the attention splits each row's ascending
 * route list at multiples of W key IDs, W = the largest power of two with
 * W * 4 * D <= 4 MiB (doubled until P = ceil(S_kv / W) <= 63; the split
 * runs when P >= 5), and gathers one key range at a time on every XCD.  Its
 * workspace holds, 256-B aligned each:
 *   range starts     int32 [B*S_q][P + 1]: for row r, entry p is the first
 *                    list position whose ID lies in range p or later, and
 *                    entry P the row's count;
 *   partial outputs  bf16 [R][Hkv][P][G][D], R = rows per pass;
 *   partial sums     fp32 [R][Hkv][P][G] (log2 of each partial's softmax
 *                    sum against its maximum score, log2 domain);
 *   with more than one pass, a second set of partial outputs and sums
 *   (each pass's partials are merged while the next pass gathers into the
 *   other set).
 * The rows are processed in passes of R rows, from the last rows to the
 * first: R = every row when one set for all of them fits, else as many
 * multiples of 4 as two sets fit (at least 256); the recommended size takes
 * R = min(B*S_q, 8192).  Results do not depend on R.
 * Returns 0 as well when a size is out of range.
 */
size_t qsa_attention_workspace_size(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D,
                                    int64_t K);

/*
 * qsa_forward_workspace_size -- recommended bytes of device workspace for
 * qsa_forward: the compacted lists and counts (4*B*S_q*K and 4*B*S_q bytes,
 * each 256-B aligned), followed by the attention's workspace
 * (qsa_attention_workspace_size).  Returns 0 when a size is out of range.
 */
size_t qsa_forward_workspace_size(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D,
                                  int64_t K);

/*
 * qsa_forward -- route-sparse GQA attention, BF16 in and out, fp32 softmax.
 *
 * Definition (flex_qsa page, `flex_sparse_gqa_attention`; fa4_qsa page,
 * `fa4_sparse_gqa_attention`; qsa page, `gathered_qsa_gqa_attention`): for
 * each (b, i, h) with hk = h / G and R = R(b,i) computed with
 * kv_length = S_kv:
 *   s_j = scale * <q[b,i,h,:], k[b,j,hk,:]>  for j in R,
 *   out[b,i,h,:] = sum_j softmax(s)_j * v[b,j,hk,:],  or +0.0 when R is empty.
 *
 *   q        [B, S_q, Hq, D] bf16; k, v [B, S_kv, Hkv, D] bf16.  Strides in
 *            elements; the last stride must be 1, base pointers 16-B
 *            aligned and the other strides multiples of 8 elements.
 *   routes   as in qsa_preprocess, in K/V coordinates of the same batch row.
 *   D        64, 128 or 256.  G = Hq / Hkv <= 16.
 *   scale    finite and > 0 (the pages default to 1/sqrt(D); callers pass it).
 *   out      OUT [B, S_q, Hq, D] bf16, contiguous, must not overlap any input
 *            or the workspace.
 *   workspace, workspace_bytes   device scratch, 256-B aligned,
 *            overwritten each call: the compacted lists and counts, then
 *            the attention's workspace; qsa_forward_workspace_size(...)
 *            bytes are recommended, and the lists plus the attention's
 *            smallest pass suffice (see qsa_attention_workspace_size).
 *
 * Runs the route-normalisation kernel into the workspace, then the
 * gather-attention kernel(s).  Errors: NULL_POINTER, EMPTY_DIM, KV_LENGTH
 * (S_kv > 2^31), HEADS, HEAD_DIM, ROUTE_DTYPE, SCALE, LAYOUT, ALIAS,
 * WORKSPACE, LIMIT, HIP.
 */
int qsa_forward(const void *q, const int64_t q_strides[4], const void *k, const int64_t k_strides[4],
                const void *v, const int64_t v_strides[4], const void *routes, int routes_dtype,
                const int64_t route_strides[3], int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq,
                int64_t Hkv, int64_t D, int64_t K, float scale, void *out, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * qsa_forward_noalloc -- qsa_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  It takes no workspace and calls no allocating
 * routine: its workspace is a device array of QSA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) built into the library, which each GPU the library runs on holds
 * until the process ends (its address is looked up on the first call on
 * each device).
 *
 * Arguments, results and errors as for qsa_forward (the same kernels run,
 * with identical results), except:
 *   - the call must fit the scratch: the compacted lists and counts
 *     (4*B*S_q*K + 4*B*S_q bytes, each 256-B aligned) plus, when the
 *     attention splits its key range, the range starts and the partial
 *     results of its smallest pass (one pass of every row, or two sets of
 *     256 rows: qsa_attention_workspace_size); larger calls return
 *     QSA_ERR_SCRATCH_LIMIT before anything is enqueued;
 *   - `stream` must belong to the current device (QSA_ERR_HIP otherwise).
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls that overlap on one GPU (several host threads, or
 * several streams) race and must be serialised by the caller.
 */
int qsa_forward_noalloc(const void *q, const int64_t q_strides[4], const void *k, const int64_t k_strides[4],
                        const void *v, const int64_t v_strides[4], const void *routes, int routes_dtype,
                        const int64_t route_strides[3], int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq,
                        int64_t Hkv, int64_t D, int64_t K, float scale, void *out, void *stream);

/*
 * qsa_forward_preprocessed -- the gather-attention kernel alone, on lists
 * already produced by qsa_preprocess (routes reused across calls, as the
 * pages build the route mask once per layer call and reuse it: qsa page,
 * `QSARouteSelection.flex_mask` and `qsa_gqa_attention` flex_mask).
 *
 *   route_list [B, S_q, K] int32 contiguous and route_count [B, S_q] int32
 *   exactly as qsa_preprocess writes them (with kv_length = S_kv).  Counts
 *   are clamped to [0, K] and IDs to [0, S_kv) before any address is formed,
 *   so malformed lists cannot fault, but their result is unspecified.
 *   lse      OUT, nullable: [B, S_q, Hq] float32, contiguous, 4-B aligned:
 *            the natural-log log-sum-exp of each row's scaled scores,
 *            log sum_j exp(s_j) (the statistic the backward needs, fa4_qsa
 *            page: the FA4 kernel owns first-order autograd); -inf for an
 *            empty route set.  Must not overlap any other argument.
 *   workspace, workspace_bytes   device scratch, 256-B aligned, overwritten
 *            each call; NULL/0 when qsa_attention_workspace_size(...) is 0,
 *            else at least the smallest pass (WORKSPACE otherwise).
 *   Other arguments as in qsa_forward.
 *
 * Gathered K/V rows are addressed as (ID) x (token stride) from each
 * (batch, head) base: in 32 bits when K and V share a non-negative token
 * stride and (S_kv - 1) * stride * 2 + 2 * D < 2^32 bytes, in 64 bits
 * otherwise (flex_qsa page, `_membership_flat_offset`: offsets past 2^31).
 */
int qsa_forward_preprocessed(const void *q, const int64_t q_strides[4], const void *k,
                             const int64_t k_strides[4], const void *v, const int64_t v_strides[4],
                             const int32_t *route_list, const int32_t *route_count, int64_t B,
                             int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K,
                             float scale, void *out, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * qsa_backward_workspace_size -- bytes of device workspace qsa_backward
 * needs, each part 256-B aligned:
 *   delta                 4 * B*S_q*Hq
 *   row x tile bit matrix 4 * B*ceil(S_q/32)*T,  T = ceil(S_kv/64)
 *   chunk prefixes        4 * B*ceil(S_q/256)*T
 *   tile totals, starts   about 8 * B*T
 *   key segments          16 * B*S_q*min(K, T)
 *   part starts, slots    about 8 * B*T, plus 8 bytes
 *   partial sums          512*D * Hkv * 2*min(P, ceil(B*S_q*min(K, T)/64)),
 *                         P = max(1, 4096 / Hkv)  (at most 1 GiB at D = 256)
 *   when dq takes the key-range split (the forward's rule, see
 *   qsa_attention_workspace_size, with Pr ranges):
 *   range starts          4 * B*S_q*(Pr + 1)
 *   dq partial sums       4 * R*Hq*Pr*D, R = min(B*S_q, 4096) rows per pass,
 *                         twice when R < B*S_q (a pass's sums are added up
 *                         while the next pass fills the other buffer)
 * Returns 0 when a size is < 1 or beyond the library's int32 segment
 * indexing (more than 2^31 - 1 segments or chunk prefixes).
 */
size_t qsa_backward_workspace_size(int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D,
                                   int64_t K);

/*
 * qsa_backward -- first-order gradients of qsa_forward, BF16 in and out,
 * fp32 arithmetic, deterministic (bitwise-repeatable for equal inputs).
 *
 * Definition (fa4_qsa page: FA4 owns first-order autograd; flex_qsa page,
 * module description: rows whose routes are all invalid have zero output and
 * zero gradients): for each (b, i, h) with hk = h / G, R = R(b,i) non-empty
 * and p = softmax over j in R of s_j = scale <q[b,i,h], k[b,j,hk]>:
 *   dp_j = <dout[b,i,h], v[b,j,hk]>,   ds_j = p_j (dp_j - <dout[b,i,h], out[b,i,h]>),
 *   dq[b,i,h]    = scale sum_j ds_j k[b,j,hk],
 *   dk[b,j,hk]  += scale ds_j q[b,i,h],   dv[b,j,hk] += p_j dout[b,i,h],
 * summed over every (i, h) whose route set holds j.  Rows with an empty R get
 * dq = +0.0 and add nothing; keys that no row routes get dk = dv = +0.0.
 *
 *   q, k, v       as in qsa_forward.
 *   out           [B, S_q, Hq, D] bf16 contiguous: this forward's output.
 *   dout          [B, S_q, Hq, D] bf16, strides as for q (last stride 1).
 *   lse           [B, S_q, Hq] float32 contiguous: the forward's lse output.
 *   route_list, route_count   as for qsa_forward_preprocessed.
 *   dq            OUT [B, S_q, Hq, D] bf16 contiguous.
 *   dk, dv        OUT [B, S_kv, Hkv, D] bf16 contiguous.
 *   workspace, workspace_bytes   device scratch of at least
 *                 qsa_backward_workspace_size(B, S_q, S_kv, Hq, Hkv, D, K) bytes,
 *                 256-B aligned (overwritten each call).
 * Outputs and workspace must not overlap each other or any input.
 *
 * Runs the dq kernel (which also forms <dout, out> per row and head), the
 * key-segment construction and the dk/dv kernel, in that order on `stream`.
 * Errors: NULL_POINTER, EMPTY_DIM, KV_LENGTH, HEADS, HEAD_DIM, SCALE,
 * LAYOUT, ALIAS, WORKSPACE, LIMIT, HIP.
 */
int qsa_backward(const void *q, const int64_t q_strides[4], const void *k, const int64_t k_strides[4],
                 const void *v, const int64_t v_strides[4], const void *out, const void *dout,
                 const int64_t dout_strides[4], const float *lse, const int32_t *route_list,
                 const int32_t *route_count, int64_t B, int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv,
                 int64_t D, int64_t K, float scale, void *dq, void *dk, void *dv, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code (never NULL). */
/*
 * qsa_select_workspace_size -- bytes of fp32 score workspace with which
 * qsa_select_token_ids scores every query row in one pass:
 * rows_rounded * ld * 4, ld = round_up(floor((q_offset + S_q) / c), 64),
 * rows_rounded = B * S_q rounded up to whole row tiles (16 rows for H <= 16,
 * 8 for H <= 32, 4 for H <= 64).  Any workspace of at least one row tile
 * (tile_rows * ld * 4 bytes) also works: the rows are then processed in
 * passes of as many whole tiles as fit, in order, on the same stream.
 * Returns 0 when an argument is out of range.
 */
size_t qsa_select_workspace_size(int64_t B, int64_t S_q, int64_t H, int64_t q_offset, int64_t compress_ratio);

/*
 * qsa_select_chunk_workspace_size -- bytes of score workspace with which
 * qsa_select_token_ids processes its query rows in passes of at least
 * query_chunk_size rows (whole row tiles; the qsa page's `query_chunk_size`
 * of `select_qsa_token_ids`, which bounds memory and changes no result):
 * min(ceil(query_chunk_size / tile_rows) * tile_rows * ld * 4, the one-pass
 * size of qsa_select_workspace_size), tile_rows and ld as there.
 * Returns 0 when an argument is out of range or query_chunk_size < 1.
 */
size_t qsa_select_chunk_workspace_size(int64_t B, int64_t S_q, int64_t H, int64_t q_offset, int64_t compress_ratio,
                                       int64_t query_chunk_size);

/*
 * qsa_select_token_ids -- route selection by compressed-block scores: the
 * producer of the routes the attention entry points consume.
 *
 * Definition (qsa page, `select_qsa_token_ids`; the page's indexer class for
 * the output width token_budget + compress_ratio - 1): local query row i
 * stands at global position t = q_offset + i (q_offset = cp_rank * S_q under
 * contiguous context parallelism, 0 otherwise).  With c = compress_ratio and
 * kb = token_budget / c (integer division):
 *   - t >= seq_lens[b] (a right-padding query): every slot is -1;
 *   - otherwise the nv = floor((t+1)/c) complete blocks are visible and block
 *     j scores sum_h relu(<index_q[b,i,h,:], block_k[b,j,0,:]>) / sqrt(D);
 *     the m = min(kb, nv) best blocks are kept, equal scores going to the
 *     smaller block index (a reading; the page fixes no tie rule);
 *   - slots [0, m*c): the kept blocks in ascending order (a reading), each as
 *     its c token IDs j*c .. j*c+c-1; slots [m*c, token_budget): -1;
 *   - slots [token_budget, token_budget + c - 1): the tokens nv*c .. t of the
 *     incomplete causal tail (0 to c-1 of them), then -1.
 * Scores are computed with bf16 products and fp32 sums and compared in fp32
 * (the page scores in an fp32 tensor).  IDs are global token positions.
 *
 *   index_q     [B, S_q, H, D] bf16 (normalised, rotated index queries),
 *               last stride 1, rows 16-B aligned, other strides multiples of 8.
 *   block_k     [B, n_blocks, 1, D] bf16 (pooled, normalised, rotated block
 *               keys), same layout rules; n_blocks >= floor(S_global / c);
 *               the size-1 head dimension's stride is ignored.
 *   seq_lens    [B] int64 right-padded logical lengths in global positions,
 *               read on the device (values outside [0, S_global] behave as
 *               clamped to it).
 *   S_global    padded global sequence length: q_offset + S_q <= S_global.
 *   D in {64, 128, 256}; 1 <= H <= QSA_MAX_INDEX_HEADS;
 *   kb <= QSA_MAX_SELECT_BLOCKS; floor(S_global / c) <= QSA_MAX_VISIBLE_BLOCKS.
 *   out         OUT [B, S_q, token_budget + c - 1] int32, contiguous.
 *   workspace   device memory of at least one row tile (see
 *               qsa_select_workspace_size), 256-B aligned; may be NULL when
 *               no row sees more than kb blocks.
 * Errors: NULL_POINTER, EMPTY_DIM, SELECTION, HEAD_DIM, LAYOUT, ALIAS,
 * WORKSPACE, LIMIT, HIP.
 */
int qsa_select_token_ids(const void *index_q, const int64_t q_strides[4], const void *block_k,
                         const int64_t k_strides[4], const int64_t *seq_lens, int64_t B, int64_t S_q, int64_t H,
                         int64_t D, int64_t S_global, int64_t q_offset, int64_t token_budget, int64_t compress_ratio,
                         int32_t *out, void *workspace, size_t workspace_bytes, void *stream);

const char *qsa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
