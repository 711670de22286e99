/*
 * misa.h — C ABI of the MISA routed token indexer for AMD Instinct MI355X (gfx950).
 *
 * The library implements the indexer of DeepSeek-Sparse-Attention-style
 * inference as described on the MISA pages (arXiv 2605.07363, "MISA: Mixture of
 * Indexer Sparse Attention for Long-Context LLM Inference": the abstract, and
 * gist.science's "Technische Samenvatting" with its sections "Probleemstelling",
 * "Methodologie: MISA" and "Hiërarchische Variant (MISA†)"):
 *
 *   1. mean-pool the indexer keys into blocks of B tokens      (misa_pool_keys)
 *   2. a router scores all H heads on the pooled keys and keeps
 *      the top-h heads of each query                           (misa_route)
 *   3. only the routed heads score every visible prefix token,
 *      S[t][s] = sum_{g in R_t} w[t][g] * max(q[t][g] . k[s], 0),
 *      and a per-query top-k keeps the selected tokens         (misa_score_topk)
 *   4. MISA†: the routed pass keeps k' candidates, the dense
 *      H-head indexer re-ranks them to the final k              (misa_hier_rerank)
 *   5. the dense DSA indexer, all H heads                      (dsa_index_dense)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers to caller-owned memory. The library
 *    never retains, frees or allocates them, and allocates no device memory at
 *    run time: scratch space is the caller's workspace `ws` of at least
 *    misa_workspace_bytes(...) bytes (256-byte aligned). A workspace may be
 *    reused by later calls on the same stream; calls that overlap in time must
 *    not share one. (misa_hier_indexer_noalloc instead uses a fixed device
 *    array that the library holds per GPU; see there.)
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *    stream). Work is enqueued asynchronously on it; no call synchronizes.
 *  - Layouts (row-major, contiguous):
 *      q      bf16  [T][H][d]        per-head indexer queries
 *      w      fp32  [T][H]           per-head weights
 *      k      bf16  [nseq][Lmax][d]  one indexer key per token, shared by all heads
 *      kbar   fp32  [nseq][Lmax/B][d] means of the complete blocks of B tokens
 *      q_seq  int32 [T]              sequence of query t (0 <= q_seq < nseq)
 *      q_len  int32 [T]              visible prefix p of query t (tokens 0..p-1;
 *                                    a causal prefill query at position t has p = t+1)
 *      heads  int32 [T][h]           routed head ids, ascending
 *      idx    int32 [T][topk]        selected token ids, ascending, -1 padded
 *      score  fp32  [T][topk]        their scores (0 in padded slots); may be NULL
 *    q and k must be 16-byte aligned; other arrays 4-byte aligned.
 *  - Supported sizes: d in {32, 64, 128, 256}; 1 <= H <= 64; 1 <= h <= H;
 *    1 <= topk; T >= 0 (T = 0 is a no-op); 1 <= Lmax < 2^31; 1 <= B <= Lmax.
 *  - Ties: tokens of equal score go to the lower token index; heads of equal
 *    router importance go to the lower head id. Scores compare as reals (-0 == +0).
 *  - Device-side values the host cannot check: a query with q_seq outside
 *    [0, nseq) is treated as empty (idx all -1; routed heads 0..h-1); q_len is
 *    clamped to [0, Lmax]; a head id outside [0, H) contributes nothing.
 *  - Return value: MISA_OK (0) or a negative MISA_ERR_*. Arguments are checked
 *    before anything is enqueued; on error nothing is enqueued and
 *    misa_last_error() (thread-local) describes the problem.
 */
#ifndef MISA_H
#define MISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MISA_API __attribute__((visibility("default")))
#else
#define MISA_API
#endif

#define MISA_OK 0
#define MISA_ERR_ARG (-1)        /* a size, range or null-pointer error            */
#define MISA_ERR_ALIGN (-2)      /* a pointer is not aligned as required            */
#define MISA_ERR_WORKSPACE (-3)  /* ws is NULL or smaller than misa_workspace_bytes */
#define MISA_ERR_HIP (-4)        /* the HIP runtime refused a launch                */

/* op codes of misa_workspace_bytes */
#define MISA_OP_ROUTE 1
#define MISA_OP_SCORE_TOPK 2
#define MISA_OP_HIER_RERANK 3
#define MISA_OP_DSA_DENSE 4
#define MISA_OP_INDEXER 5
#define MISA_OP_HIER_INDEXER 6
#define MISA_OP_BLOCK_FILTER 7     /* kc argument = m, the complete blocks kept */
#define MISA_OP_BLOCK_INDEXER 8    /* kc argument = m */
#define MISA_OP_PIVOT_INDEXER 9    /* B argument = G, the group size */

/* Library version, major * 10000 + minor * 100 + patch. */
MISA_API int32_t misa_version(void);

/* Human-readable name of a status code (static storage). */
MISA_API const char* misa_status_string(int32_t code);

/* Message describing the last error returned on the calling thread ("" if none). */
MISA_API const char* misa_last_error(void);

/*
 * Workspace bytes needed by one call of `op` (MISA_OP_*) with these sizes.
 * Arguments that an op does not use are ignored (kc matters for the MISA†
 * ops, and stands for m, the blocks kept, in the block ops; B for the ops that
 * route or pool). Returns 0 if none is needed.
 * The scoring ops hold fp32 score rows for at most 1 GiB of queries at a time
 * (min(T, 2^28 / Lmax) rows): a larger batch, such as a long causal prefill, is
 * scored and selected in consecutive slabs of queries on the stream, so the
 * workspace does not grow with T * Lmax beyond that bound. misa_indexer and
 * misa_hier_indexer run their fused decode pipeline (score rows for the whole
 * batch) only for batches of at most 4096 queries; larger batches take the
 * separate calls and their bound.
 */
MISA_API size_t misa_workspace_bytes(int32_t op, int64_t T, int32_t H, int64_t Lmax, int32_t B, int32_t topk,
                            int32_t kc);

/*
 * Block mean-pooling of the indexer keys (MISA pages, "Methodologie: MISA":
 * the prefix is split into blocks of B tokens and the router works on
 * mean-pooled keys).
 *   k     bf16 [nseq][Lmax][d]    in
 *   kbar  fp32 [nseq][Lmax/B][d]  out: kbar[n][j] = mean of k[n][jB .. jB+B-1]
 * Only complete blocks are written; a query's partial last block is pooled by
 * misa_route from k. Deterministic (fixed summation order).
 */
MISA_API int32_t misa_pool_keys(const void* k, int64_t nseq, int64_t Lmax, int32_t d, int32_t B, float* kbar,
                       void* stream);

/*
 * Incremental pooling for a decode loop. The router's O(H * M) cost
 * ("Methodologie: MISA") presumes that the pooled keys already exist; this call
 * keeps them current after tokens were appended to the key cache, by pooling
 * only the blocks that the append completed.
 *   k         bf16 [nseq][Lmax][d]    in, already holding the appended keys
 *   prev_len  int32 [nseq]            in: tokens of each sequence before the append
 *   new_len   int32 [nseq]            in: tokens after it
 *   max_new   bound on new_len[n] - prev_len[n] over the batch (0 .. Lmax)
 *   kbar      fp32 [nseq][Lmax/B][d]  in/out: kbar[n][j] is rewritten for every
 *             block j with prev_len[n] < (j + 1) B <= new_len[n]; every other
 *             block keeps its value
 * The written means are bit-identical to what misa_pool_keys writes for the
 * same blocks. A sequence whose pair is not an append (prev_len < 0,
 * new_len < prev_len or new_len > Lmax) is left alone; blocks completed
 * beyond max_new new tokens are not pooled (max_new must bound the append).
 * Errors: MISA_ERR_ARG (sizes, max_new outside [0, Lmax], null pointers),
 * MISA_ERR_ALIGN (k, kbar not 16-byte or the lengths not 4-byte aligned).
 */
MISA_API int32_t misa_pool_update(const void* k, int64_t nseq, int64_t Lmax, int32_t d, int32_t B,
                                  const int32_t* prev_len, const int32_t* new_len, int32_t max_new, float* kbar,
                                  void* stream);

/*
 * Block-pooled MoE router (MISA abstract; "Methodologie: MISA": per-head
 * affinities with pooled keys over M = ceil(p/B) blocks, aggregated into one
 * importance per head, top-h heads kept; cost O(H * M)).
 * Importance of head g for query t (the last block may be partial: its mean is
 * over the tokens the query sees):
 *     r[t][g] = w[t][g] * sum_{j < ceil(p/B)} max(q[t][g] . Kbar_j, 0)
 *   q, w, k, kbar, q_seq, q_len   in (kbar from misa_pool_keys with the same B)
 *   heads       int32 [T][h]  out: the h heads of largest r, ascending id
 *   router_key  fp32  [T][H]  out (may be NULL): r[t][g]
 *   ws / ws_bytes             workspace, misa_workspace_bytes(MISA_OP_ROUTE, T, H, Lmax, B, 0, 0)
 */
MISA_API int32_t misa_route(const void* q, const float* w, const void* k, const float* kbar, const int32_t* q_seq,
                   const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax,
                   int32_t B, int32_t h, int32_t* heads, float* router_key, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * Routed token scoring + per-query top-k (MISA abstract; "Methodologie: MISA",
 * sparse token scoring: only the h routed heads score every prefix token; the
 * final top-k comes from these reduced scores):
 *     S[t][s] = sum_{g in heads[t]} w[t][g] * max(q[t][g] . k[q_seq[t]][s], 0),  s < q_len[t]
 *   heads   int32 [T][h]   in (from misa_route, or any ids in [0, H))
 *   idx     int32 [T][topk] out: the topk best s (ties: lower s), ascending, -1 padded;
 *                           a query with q_len <= topk gets all of its prefix
 *   score   fp32  [T][topk] out (may be NULL)
 *   ws / ws_bytes           misa_workspace_bytes(MISA_OP_SCORE_TOPK, T, H, Lmax, 0, topk, 0)
 * With topk = k' this is the coarse pass of MISA† (its idx is the candidate set).
 */
MISA_API int32_t misa_score_topk(const void* q, const float* w, const void* k, const int32_t* heads, int32_t h,
                        const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                        int64_t nseq, int64_t Lmax, int32_t topk, int32_t* idx, float* score, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Fine stage of MISA† ("Hiërarchische Variant (MISA†)": the dense DSA indexer,
 * all H heads, re-scores only the k' candidates of the routed pass and keeps the
 * final top-k).
 *   cand   int32 [T][kc]  in: candidate token ids, ascending, -1 padded (the idx
 *                          output of misa_score_topk with topk = kc). Entries
 *                          outside [0, q_len) are not candidates; each valid
 *                          entry is scored once per occurrence.
 *   idx    int32 [T][topk] out: the topk candidates of best dense score (ties:
 *                          lower candidate slot, i.e. lower token id for an
 *                          ascending list), in candidate-slot order (ascending
 *                          token id), -1 padded when fewer than topk are valid
 *   score  fp32  [T][topk] out (may be NULL): their dense scores
 *   Requires kc >= topk.  ws: misa_workspace_bytes(MISA_OP_HIER_RERANK, T, H, Lmax, 0, topk, kc)
 */
MISA_API int32_t misa_hier_rerank(const void* q, const float* w, const void* k, const int32_t* cand, int32_t kc,
                         const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                         int64_t nseq, int64_t Lmax, int32_t topk, int32_t* idx, float* score, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * Dense DSA indexer (MISA abstract; "Probleemstelling": the DSA indexer scores
 * every prefix token with all H_I heads and keeps the top-k, shared by all
 * heads). misa_score_topk with heads = {0..H-1}; the same summation order, so a
 * routed call with h = H and heads 0..H-1 returns bit-identical results.
 *   ws: misa_workspace_bytes(MISA_OP_DSA_DENSE, T, H, Lmax, 0, topk, 0)
 */
MISA_API int32_t dsa_index_dense(const void* q, const float* w, const void* k, const int32_t* q_seq,
                        const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax,
                        int32_t topk, int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole MISA indexer in one call: misa_route followed by misa_score_topk
 * (MISA abstract; "Methodologie: MISA"), with bit-identical results. For decode
 * shapes (fewer than 8 queries per sequence on average) it runs as one pipeline
 * of four launches: router partials, head selection fused into the routed
 * scoring, and a two-launch top-k; otherwise it makes the separate calls.
 *   kbar     fp32 [nseq][Lmax/B][d] from misa_pool_keys (the pooled-key cache)
 *   heads    int32 [T][h] out, may be NULL: the routed heads
 *   idx / score as misa_score_topk
 *   ws: misa_workspace_bytes(MISA_OP_INDEXER, T, H, Lmax, B, topk, 0)
 */
MISA_API int32_t misa_indexer(const void* q, const float* w, const void* k, const float* kbar, const int32_t* q_seq,
                              const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax,
                              int32_t B, int32_t h, int32_t topk, int32_t* heads, int32_t* idx, float* score,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * The whole MISA† indexer in one call: misa_route, misa_score_topk with
 * topk = kc (the enlarged candidate set) and misa_hier_rerank to topk
 * ("Hiërarchische Variant (MISA†)"), with bit-identical results. For decode
 * shapes it runs as six launches, the candidates' dense re-scoring fused into
 * the coarse pass's compaction.
 *   heads  int32 [T][h] out, may be NULL;  cand  int32 [T][kc] out, may be NULL
 *   ws: misa_workspace_bytes(MISA_OP_HIER_INDEXER, T, H, Lmax, B, topk, kc)
 */
MISA_API int32_t misa_hier_indexer(const void* q, const float* w, const void* k, const float* kbar,
                                   const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                                   int64_t nseq, int64_t Lmax, int32_t B, int32_t h, int32_t kc, int32_t topk,
                                   int32_t* heads, int32_t* cand, int32_t* idx, float* score, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * misa_hier_indexer for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. It
 * takes no workspace argument and allocates nothing; its scratch is a device
 * array of MISA_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends. The caller still passes the inputs and outputs, with
 * the meaning, layout and results of misa_hier_indexer (same kernels, bit for
 * bit).
 *  - Sizes whose workspace (misa_workspace_bytes(MISA_OP_HIER_INDEXER, ...))
 *    exceeds MISA_SCRATCH_BYTES are refused with MISA_ERR_WORKSPACE before
 *    anything is enqueued (decode batches fit: 4 x 128K tokens need about
 *    9 MiB; a long causal prefill does not).
 *  - The scratch belongs to the GPU of `stream` (NULL: the current device). Its
 *    address is looked up once per device, on the first call there. Every call
 *    on a GPU shares that GPU's array and leaves its contents behind; each call
 *    clears, with its own kernels, the state it needs zeroed. Calls that overlap
 *    in time on one GPU (other streams, other host threads) race on the array
 *    and must be serialized by the caller.
 * Errors: as misa_hier_indexer; MISA_ERR_HIP if the scratch address cannot be
 * obtained.
 */
#define MISA_SCRATCH_BYTES (32u << 20)
MISA_API int32_t misa_hier_indexer_noalloc(const void* q, const float* w, const void* k, const float* kbar,
                                           const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H,
                                           int32_t d, int64_t nseq, int64_t Lmax, int32_t B, int32_t h, int32_t kc,
                                           int32_t topk, int32_t* heads, int32_t* cand, int32_t* idx, float* score,
                                           void* stream);

/*
 * Block filter on the pooled keys, composed with head routing: the coarse stage
 * of a two-stage (block, then token) search. HISA (thelatestinai.com paper
 * cards, the HISA abstract) scores pooled block representations, drops the
 * weak blocks and runs the indexer only inside the retained ones; the
 * gist.science MISA summary presents head routing as combinable with such
 * token-axis schemes ("Betekenis en Claims"). The pages give no formula for the
 * coarse score; this library takes the routed indexer formula on the block's
 * mean key, b_j = sum over the routed heads g of w[t][g] * max(q[t][g] . kbar[j], 0),
 * for the complete visible blocks j < q_len[t] / B, keeps the m best (ties to
 * the lower block id; all of them when there are at most m) and always keeps
 * the partial last block.
 *   kbar    fp32 [nseq][Lmax/B][d]  from misa_pool_keys
 *   heads   int32 [T][h]            routed heads (an id outside [0, H) contributes nothing)
 *   m       complete blocks kept per query, 1 .. Lmax / B
 *   blocks  int32 [T][m] out: kept complete block ids, ascending, -1 padded
 *   cand    int32 [T][(m + 1) * B] out, may be NULL: the token ids of the kept
 *           blocks, then those of the partial block, ascending, -1 padded (the
 *           candidate list of misa_hier_rerank's form, for the fine stage)
 *   ws: misa_workspace_bytes(MISA_OP_BLOCK_FILTER, T, H, Lmax, B, 0, m)
 * Errors: as misa_route, and MISA_ERR_ARG for m outside [1, Lmax / B].
 */
MISA_API int32_t misa_block_filter(const void* q, const float* w, const float* kbar, const int32_t* heads,
                                   int32_t h, const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H,
                                   int32_t d, int64_t nseq, int64_t Lmax, int32_t B, int32_t m, int32_t* blocks,
                                   int32_t* cand, void* ws, size_t ws_bytes, void* stream);

/*
 * Routed indexer restricted to the retained blocks: misa_route, then
 * misa_block_filter, then the routed scores of the candidate tokens and their
 * top-k (score descending, token id ascending; ids ascending, -1 padded). With
 * m = Lmax / B every visible token is a candidate and the result equals
 * misa_indexer's. Each query reads the keys of at most (m + 1) * B tokens.
 *   heads   int32 [T][h] out, may be NULL;  blocks  int32 [T][m] out, may be NULL
 *   idx / score as misa_score_topk (score: routed scores)
 *   ws: misa_workspace_bytes(MISA_OP_BLOCK_INDEXER, T, H, Lmax, B, topk, m)
 */
MISA_API int32_t misa_block_indexer(const void* q, const float* w, const void* k, const float* kbar,
                                    const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                                    int64_t nseq, int64_t Lmax, int32_t B, int32_t h, int32_t m, int32_t topk,
                                    int32_t* heads, int32_t* blocks, int32_t* idx, float* score, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * Proxy-query shared scan with per-query refinement (PIVOT-Refine;
 * thelatestinai.com paper cards, the PIVOT abstract). The queries are taken in
 * groups of G consecutive ones (the last group may be shorter), and every query
 * of a group must belong to the sequence of its first query (prefill: G
 * consecutive positions; decode: the positions of one multi-token step). Each
 * group is folded into a proxy query, the sum of its per-head queries rounded to
 * bf16 (nearest, ties to even) with the sum of their head weights (the page
 * leaves the fold open; the sum is the mean up to a positive factor, which
 * changes no ranking). The proxy scans its group's longest prefix once with the
 * dense indexer (all H heads) and keeps kc candidates (ties to the lower token
 * id); each query then re-ranks those candidates with its own dense indexer as
 * misa_hier_rerank does (ids at or beyond its own prefix are skipped).
 *   cand   int32 [T][kc] out, may be NULL: the candidates of each query's group
 *   idx / score as misa_hier_rerank (dense scores)
 *   ws: misa_workspace_bytes(MISA_OP_PIVOT_INDEXER, T, H, Lmax, G, topk, kc) (sized for d up to 256)
 * Errors: as misa_hier_rerank, and MISA_ERR_ARG for G < 1 or kc outside [topk, Lmax].
 */
MISA_API int32_t misa_pivot_indexer(const void* q, const float* w, const void* k, const int32_t* q_seq,
                                    const int32_t* q_len, int64_t T, int32_t H, int32_t d, int64_t nseq, int64_t Lmax,
                                    int32_t G, int32_t kc, int32_t topk, int32_t* cand, int32_t* idx, float* score,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * Full score rows of the routed scoring step (a diagnostic of step 3 above):
 * scores fp32 [T][Lmax], row t filled for s < q_len[t], other entries untouched.
 * heads may be NULL (then h must equal H: dense scores).
 */
MISA_API int32_t misa_debug_scores(const void* q, const float* w, const void* k, const int32_t* heads, int32_t h,
                          const int32_t* q_seq, const int32_t* q_len, int64_t T, int32_t H, int32_t d,
                          int64_t nseq, int64_t Lmax, float* scores, void* stream);

/*
 * Event timing of one internal kernel class, for measurement tools:
 * kernel 1 = token scoring over prefixes (routed or dense), 2 = top-k,
 * 3 = router, 4 = pooling, 5 = token scoring over candidate lists (re-rank).
 * After misa_timing_begin(kernel, capacity, stream), each launch of that kernel
 * class on `stream` (up to `capacity` launches) is bracketed by events on that
 * stream; launches on other streams are not touched. misa_timing_end(stream,
 * ...) waits for the recorded events, returns the summed duration in ms and
 * the number of launches timed, and ends the timing of that stream. A second
 * begin on a stream replaces the first. While no stream is timed the launch
 * hooks cost one atomic load. Beginning or ending the timing of a stream while
 * another thread launches on that same stream is not supported.
 */
MISA_API int32_t misa_timing_begin(int32_t kernel, int32_t capacity, void* stream);
MISA_API int32_t misa_timing_end(void* stream, float* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MISA_H */
