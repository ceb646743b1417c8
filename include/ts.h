/*
 * ts.h -- C ABI of the TokenSwift-style verify/draft attention and dynamic
 * partial-KV-cache kernels for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute follows the TokenSwift pages:
 *   - tool listing, "How it works": verification runs the target model once
 *     over all drafts (a candidate tree plus retrieved 4-grams) against the
 *     COMPLETE KV cache, each draft seeing only its own tree ancestors;
 *     drafting runs the target model itself, with a small set of extra linear
 *     heads, over a REDUCED (partial) KV cache and proposes 4 tokens per pass;
 *   - summary page, "Approach": the reduced cache is re-selected during
 *     generation by how strongly queries attend to its keys;
 *   - model card, command-line example: retrieval budget 4096 tokens, gamma 4,
 *     ngram_topk 20, generation up to 102400 tokens.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory and keeps no state besides a thread-local
 *     error message. Scratch space is passed in as `workspace`.
 *   - Element type `ts_dtype`: TS_BF16 (uint16 bit patterns of bfloat16) or
 *     TS_F32. Accumulation is always fp32. Outputs of attention are written in
 *     the input type (bf16 rounded to nearest even); LSE and scores in fp32.
 *   - Layouts are row-major and dense in the last dimension, e.g. q[T][Hq][D]
 *     means element (t, h, d) at q + (t*Hq + h)*D + d.
 *   - GQA: query head h reads KV head h / (Hq/Hkv) (contiguous groups).
 *   - Tensor pointers must be 16-byte aligned; D must be 64 or 128.
 *   - Every call validates its arguments on the host and returns a non-zero
 *     ts_status BEFORE launching anything when they are bad; ts_last_error()
 *     then describes the problem. On success the work is only enqueued on
 *     `stream` (asynchronous); faults surface at the caller's next sync.
 *   - Calls are re-entrant. Two calls that share a workspace must be ordered
 *     (same stream, or synchronised).
 */
#ifndef TS_H_
#define TS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ts_status {
  TS_OK = 0,
  TS_ERR_INVALID_ARG = 1, /* null/misaligned pointer, inconsistent sizes    */
  TS_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels handle  */
  TS_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returns  */
  TS_ERR_HIP = 4          /* a HIP launch failed; message from the runtime  */
} ts_status;

/* Element type of the tensors of a call. A call given any other value returns
 * TS_ERR_INVALID_ARG; the last enumerator only widens the type to the range of
 * an int, so that such a value is a valid ts_dtype in C++ as in C. */
typedef enum ts_dtype { TS_F32 = 0, TS_BF16 = 1, TS_DTYPE_INT_RANGE_ = 0x7fffffff } ts_dtype;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ts_last_error(void);

/* ABI version of this header (bumped on any signature change). */
int ts_abi_version(void);

#define TS_ABI_VERSION 3
#define TS_MAX_DRAFT 1024 /* max draft tokens T of one verify call */

/* ------------------------------------------------------------------------
 * Tree-verify attention (tool listing, "How it works": one verification pass
 * of the target model over all drafts against the complete cache, with the
 * tree mask).
 *
 * For draft row t in [0,T), query head h, g = h / (Hq/Hkv):
 *   A(t) = {t} + ancestors of t along parent[]      (ancestor-or-self mask)
 *   keys  = cached tokens j in [0, L) of head g  +  draft tokens a in A(t)
 *   s     = scale * <q[t,h], k>
 *   out[t,h] = softmax(s) . v          lse[t,h] = ln sum exp(s)   (natural log)
 *
 *   q        [T][Hq][D]                  draft queries (already position-encoded)
 *   k_cache  [Hkv][cache_stride][D]      rows [0, L) are read; cache_stride >= L
 *   v_cache  same layout as k_cache
 *   k_draft  [Hkv][T][D]                 K/V of the T drafts (not yet in the cache)
 *   v_draft  [Hkv][T][D]
 *   parent   int32 [T] on the device, parent[t] in [-1, t); -1 marks a root, so
 *            forests (tree + independent 4-gram chains) are allowed. Entries
 *            outside [-1, t) are treated as -1 (never read out of bounds).
 *   out      [T][Hq][D]   written in `dtype`
 *   lse      [T][Hq] fp32, may be NULL
 *   scale    softmax scale (usually 1/sqrt(D)); finite and > 0, else
 *            TS_ERR_INVALID_ARG
 *   num_splits  0 = library choice; otherwise the number of key ranges the
 *            work is split into (results agree across choices up to rounding).
 *            Must match the value given to the size query.
 *   workspace   >= ts_tree_verify_attn_workspace(...) bytes, 256-byte aligned;
 *            contents on entry are ignored. It holds the split partials: each
 *            split's normalised output in the input dtype (bf16 inputs: bf16,
 *            rounded to nearest even; fp32 inputs: fp32) and its fp32 lse.
 * Supported: T in [1, 1024], Hq in [1, 4096], Hq % Hkv == 0, Hq/Hkv <= 16,
 *            D in {64, 128}, 0 <= L <= 2^30, and one launch's worth of
 *            (split, KV head, row group) units (TS_ERR_UNSUPPORTED beyond).
 * ---------------------------------------------------------------------- */
size_t ts_tree_verify_attn_workspace(int T, int Hq, int Hkv, int D, int64_t L,
                                     ts_dtype dtype, int num_splits);

ts_status ts_tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                              int64_t cache_stride, const void* k_draft, const void* v_draft,
                              const int32_t* parent, void* out, float* lse,
                              int T, int Hq, int Hkv, int D, int64_t L, float scale,
                              ts_dtype dtype, int num_splits,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ts_tree_verify_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, results and checks as
 * ts_tree_verify_attn, minus the workspace: the split partials go to a static
 * device array of TS_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends. A call whose partials
 * (ts_tree_verify_attn_workspace(...) bytes) exceed it returns
 * TS_ERR_UNSUPPORTED before any HIP call. The stream must belong to the
 * current device; the first call on a device looks its array up (no
 * allocation). All calls on one GPU share the array: calls that overlap on one
 * GPU (other streams, other threads) race and must be ordered by the caller. */
#define TS_NOALLOC_SCRATCH_BYTES (64u << 20)

ts_status ts_tree_verify_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      int64_t cache_stride, const void* k_draft, const void* v_draft,
                                      const int32_t* parent, void* out, float* lse,
                                      int T, int Hq, int Hkv, int D, int64_t L, float scale,
                                      ts_dtype dtype, int num_splits, hipStream_t stream);

/* The two phases of ts_tree_verify_attn, for callers that merge partial
 * results themselves (e.g. partials computed on several devices, each over
 * its own slice of the cache -- merging across devices is the same log-sum-
 * exp rule as merging across splits).
 *
 * ts_tree_verify_attn_partials writes, for every split s in [0, n_splits):
 *   o_part [n_splits][T][Hq][D]  part_dtype   softmax(s restricted to split s) . v
 *   l_part [n_splits][T][Hq]     fp32         ln sum exp(s) over split s (-inf if empty)
 * with n_splits = ts_tree_verify_attn_num_splits(...). part_dtype is TS_F32,
 * or TS_BF16 (rounded to nearest even: half the bytes for the merge to read)
 * when dtype is TS_BF16; else TS_ERR_UNSUPPORTED. Split s covers a
 * contiguous range of cached tokens; the draft tokens belong to the last split.
 * ts_attn_merge combines `n_parts` such partials:
 *   lse = ln sum_s exp(l_part[s]);  out = sum_s exp(l_part[s] - lse) * o_part[s]. */
int ts_tree_verify_attn_num_splits(int T, int Hq, int Hkv, int D, int64_t L,
                                   ts_dtype dtype, int num_splits);

ts_status ts_tree_verify_attn_partials(const void* q, const void* k_cache, const void* v_cache,
                                       int64_t cache_stride, const void* k_draft,
                                       const void* v_draft, const int32_t* parent,
                                       void* o_part, ts_dtype part_dtype, float* l_part,
                                       int T, int Hq, int Hkv, int D, int64_t L, float scale,
                                       ts_dtype dtype, int num_splits, hipStream_t stream);

/* o_part in part_dtype (TS_F32 or TS_BF16); out in dtype. */
ts_status ts_attn_merge(const void* o_part, ts_dtype part_dtype, const float* l_part, int n_parts,
                        int rows, int D, void* out, float* lse, ts_dtype dtype,
                        hipStream_t stream);

/* ts_tree_verify_attn_partials followed by ts_kv_importance_score over the
 * same cache, in one launch where the shapes allow. In a decode step the
 * verification pass reads the whole cache of a layer and the partial-cache
 * refresh scores that same cache's chunks against the latest queries (tool
 * listing, "How it works"; summary page, "Approach"): one pass over K can
 * serve both. The arguments are those of ts_tree_verify_attn_partials, then
 * those of ts_kv_importance_score that differ (q_recent [R][Hq][D], R, chunk,
 * imp_scale, scores [Hkv][L/chunk]), with the same meaning, layout, checks and
 * errors; the importance is taken over k_cache rows [0, L). Results are those
 * of the two calls (o_part, l_part bit-identical; scores equal up to fp32
 * summation order). One launch when dtype is bf16, D = 128, chunk = 64,
 * L % 64 == 0, T <= 256, Hq/Hkv is 1, 2 or 4 with R*(Hq/Hkv) <= 32, and the
 * verify rows of a KV head (T*Hq/Hkv, above 128) leave the last 32 of their
 * last 256-row group empty (e.g. 480 rows); otherwise the two launches. */
ts_status ts_tree_verify_attn_partials_and_importance(
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_stride, const void* k_draft,
    const void* v_draft, const int32_t* parent, void* o_part, ts_dtype part_dtype, float* l_part, int T, int Hq,
    int Hkv, int D, int64_t L, float scale, ts_dtype dtype, int num_splits, const void* q_recent, int R, int chunk,
    float imp_scale, float* scores, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Chunk importance (summary page, "Approach": the reduced cache is chosen by
 * how strongly queries attend to its keys). For KV head g and chunk
 * c = tokens [c*chunk, (c+1)*chunk):
 *   u[r, j]     = max over query heads h of group g of  scale * <q_recent[r,h], k[g,j]>
 *   scores[g,c] = mean over r in [0,R) and j in chunk c of u[r, j]
 * (max over the grouped heads, mean over tokens and recent queries: the pages
 * name the importance but not its reduction; this is the reading used.)
 *
 *   q_recent [R][Hq][D]            the R most recent queries (R = gamma = 4)
 *   k_cache  [Hkv][cache_stride][D] rows [0, L) read; V is never read
 *   scores   [Hkv][L/chunk] fp32
 * Supported: L % chunk == 0, chunk in [1, 4096], R*(Hq/Hkv) <= 64,
 * Hq/Hkv <= 16, D in {64,128}.
 * ---------------------------------------------------------------------- */
ts_status ts_kv_importance_score(const void* q_recent, const void* k_cache, int64_t cache_stride,
                                 float* scores, int R, int Hq, int Hkv, int D, int64_t L,
                                 int chunk, float scale, ts_dtype dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ts_attn_merge followed by ts_kv_importance_score, in one launch where the
 * shapes allow. In a decode step the verify pass's merge and the partial-KV
 * refresh's chunk importance depend on nothing of each other, so both can run
 * as one grid: its first workgroups merge rows, the others score chunks, each
 * with its own kernel's code. The results are bit-identical to the two calls.
 * This is a launch-level variant of those two operations (model card CLI
 * example and summary page "Approach": verification of the drafts and the
 * dynamic partial cache), not an operation of its own.
 *
 * Arguments: those of ts_attn_merge (o_part .. out_dtype, with Dv its D and
 * out_dtype its dtype), then those of ts_kv_importance_score, with the same
 * meaning, layout, checks and errors. The two operations' buffers must not
 * overlap. One launch when Dv = D = 128, n_parts <= 16, dtype is bf16,
 * chunk = 64 and R*(Hq/Hkv) <= 64; otherwise the two launches of the separate
 * calls, merge first, on the same stream.
 * ---------------------------------------------------------------------- */
ts_status ts_attn_merge_and_importance(const void* o_part, ts_dtype part_dtype, const float* l_part, int n_parts,
                                       int rows, int Dv, void* out, float* lse, ts_dtype out_dtype, const void* q_recent,
                                       const void* k_cache, int64_t cache_stride, float* scores, int R, int Hq,
                                       int Hkv, int D, int64_t L, int chunk, float scale, ts_dtype dtype,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Top-k chunk selection (model card CLI: retrieval budget 4096 tokens =
 * k chunks of `chunk` tokens). Per KV head independently: the k chunks of
 * highest score, ties broken toward the lower chunk index, written in
 * ASCENDING chunk index (so a gathered cache keeps time order).
 *   scores      [Hkv][n_chunks] fp32 (NaN not allowed)
 *   chunk_idx   [Hkv][k] int32 out
 *   chunk_score [Hkv][k] fp32 out, may be NULL (scores of the chosen chunks)
 * Supported: 1 <= k <= n_chunks <= 65536. No workspace.
 * ---------------------------------------------------------------------- */
ts_status ts_kv_topk_select(const float* scores, int Hkv, int n_chunks, int k,
                            int32_t* chunk_idx, float* chunk_score, hipStream_t stream);

/* ts_attn_merge followed by ts_kv_topk_select, in one launch where the merge
 * allows: in a decode step both depend only on the verify pass (its split
 * partials and, through ts_tree_verify_attn_partials_and_importance, the chunk
 * scores), and run as one grid whose first Hkv workgroups select chunks. The
 * arguments are those of ts_attn_merge (Dv its D), then those of
 * ts_kv_topk_select, with the same meaning, checks and errors; the two
 * operations' buffers must not overlap. Results are bit-identical to the two
 * calls. One launch when Dv = 128 and n_parts <= 16; otherwise the two
 * launches, merge first. */
ts_status ts_attn_merge_and_topk(const void* o_part, ts_dtype part_dtype, const float* l_part, int n_parts,
                                 int rows, int Dv, void* out, float* lse, ts_dtype out_dtype, const float* scores, int Hkv,
                                 int n_chunks, int k, int32_t* chunk_idx, float* chunk_score,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gather of the chosen chunks into a partial cache (summary page, "Approach").
 *   k_part[g][i*chunk + u][:] = k_cache[g][chunk_idx[g][i]*chunk + u][:]
 *   (and the same for V), bit-exact copies.
 *   k_part, v_part [Hkv][k*chunk][D]. An index outside [0, L/chunk) writes
 *   zeros for that chunk (never reads out of bounds).
 * Supported: L % chunk == 0, chunk*D*elem_size a multiple of 16 bytes.
 * ---------------------------------------------------------------------- */
ts_status ts_kv_gather(const void* k_cache, const void* v_cache, int64_t cache_stride,
                       const int32_t* chunk_idx, int Hkv, int k, int chunk, int D, int64_t L,
                       void* k_part, void* v_part, ts_dtype dtype, hipStream_t stream);

/* ts_kv_gather followed by ts_partial_draft_attn over the gathered cache, in
 * one pass where possible: the draft step refreshes the partial cache from the
 * chosen chunks (summary page, "Approach": dynamic partial-cache update) and
 * attends over it (tool listing, "How it works"); with bf16 and 64-token
 * chunks the attention reads each chosen chunk from the full cache once and
 * writes the copy on the way, instead of a separate copy pass and a second
 * read. Arguments are those of ts_kv_gather (k_cache .. v_part, with
 * Hkv, D and dtype given once below) and of ts_partial_draft_attn with
 * P = k*chunk; the same checks and errors, all made before anything runs.
 * k_part and v_part hold the gathered chunks and out / lse the draft
 * attention afterwards, bit-identical to the two calls with the same
 * num_splits (an index outside [0, L/chunk) is a zero chunk in both). The
 * partial cache must not overlap the full cache. Otherwise (fp32, other chunk
 * sizes, more than 16 query rows per KV head) the two calls are made. */
ts_status ts_kv_gather_and_draft_attn(const void* k_cache, const void* v_cache, int64_t cache_stride,
                                      const int32_t* chunk_idx, int k, int chunk, int64_t L,
                                      void* k_part, void* v_part, const void* q, const void* k_new,
                                      const void* v_new, void* out, float* lse, int Tq, int Hq, int Hkv,
                                      int D, float scale, ts_dtype dtype, int num_splits, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Draft attention over the partial cache (tool listing, "How it works":
 * drafting runs the target model itself over the reduced cache, proposing
 * 4 tokens per pass).
 * Tq new tokens attend to all P gathered tokens and causally among
 * themselves: exactly ts_tree_verify_attn with the chain parent[t] = t-1.
 *   q [Tq][Hq][D]; k_part, v_part [Hkv][P][D]; k_new, v_new [Hkv][Tq][D];
 *   out [Tq][Hq][D]; lse [Tq][Hq] fp32 (may be NULL).
 * Supported: as ts_tree_verify_attn with T = Tq.
 * ---------------------------------------------------------------------- */
size_t ts_partial_draft_attn_workspace(int Tq, int Hq, int Hkv, int D, int64_t P,
                                       ts_dtype dtype, int num_splits);

ts_status ts_partial_draft_attn(const void* q, const void* k_part, const void* v_part,
                                const void* k_new, const void* v_new, void* out, float* lse,
                                int Tq, int Hq, int Hkv, int D, int64_t P, float scale,
                                ts_dtype dtype, int num_splits,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Candidate tree of draft tokens from the per-position logits (tool listing,
 * "How it works": one pass yields logits for the next positions and the
 * candidates are organised as a tree; the summary page's ablation table uses
 * the shapes [1,3,3,3], [3,3,3,3] and [1,9,9,9]).
 *
 *   logits  [P][V] in `dtype` (TS_F32 or TS_BF16), position d in row d; NaN
 *           not allowed
 *   shape   HOST array of `depth` ints: k_d candidates at depth d
 *   Depth d's candidates are the k_d highest logits of row d, equal logits
 *   ranked by lower token id. The tree is the product of the depths: each
 *   node of depth d has k_{d+1} children. Nodes are numbered breadth-first,
 *   inside a depth in lexicographic order of the candidate ranks along the
 *   root path, so parent[t] < t and the result feeds ts_tree_verify_attn
 *   (which takes T <= 1024) directly.
 *   Written (device, int32): parent [T] (-1 for depth-0 nodes), draft_tok [T]
 *   (the node's candidate token), cand [depth][16] if not NULL (ranked
 *   candidates, -1 past k_d).
 * T = ts_draft_tree_nodes(shape, depth) = sum_d k_0*..*k_d. Workspace: at least
 * ts_build_draft_tree_workspace(V, depth) bytes, contents ignored on entry.
 * Supported: depth in [1, 8], k_d in [1, 16], k_d <= V, T <= 1024, P >= depth.
 * ---------------------------------------------------------------------- */
int ts_draft_tree_nodes(const int32_t* shape, int depth);   /* -1 if unsupported */

/* Scratch for the per-slice candidates (<= 64 KiB), 256-byte aligned; 0 on bad sizes. */
size_t ts_build_draft_tree_workspace(int V, int depth);

ts_status ts_build_draft_tree(const void* logits, int P, int V, const int32_t* shape, int depth,
                              int32_t* parent, int32_t* draft_tok, int32_t* cand, ts_dtype dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Acceptance and KV-cache commit (tool listing, "How it works": the drafts are
 * checked for an exact match with the target model's tokens, one of the
 * longest valid drafts is chosen at random, and the KV cache is updated).
 *
 *   parent      int32 [T] on the device, the draft forest of the verify call
 *               (entries outside [-1, t) count as roots)
 *   draft_tok   int32 [T] the drafts' tokens
 *   target_tok  int32 [T+1]: [0] the target's token for the position after
 *               the committed context, [t+1] its token for the position after
 *               draft t (from the verify pass at row t)
 *   rand_u32    a uniform random number drawn by the caller
 *   A root is valid when draft_tok[root] == target_tok[0]; a node a with
 *   parent p when its parent is valid and draft_tok[a] == target_tok[p+1].
 *   Among the valid nodes of greatest depth, in index order, number
 *   rand_u32 % count is chosen; n = its depth + 1 (0 if no root is valid).
 *   Written (device, int32): *n_accepted = n; path[0..n) = the chosen root
 *   path root first, path[n..T) = -1; *bonus = target_tok[last + 1]
 *   (target_tok[0] when n = 0).
 *   Commit: k_cache[g][L+i][:] = k_draft[g][path[i]][:] for i < n, every KV
 *   head g, and the same for V (bit-exact copies).
 *   k_cache, v_cache [Hkv][cache_stride][D]; k_draft, v_draft [Hkv][T][D].
 * Requires L + T <= cache_stride (room for the longest possible path).
 * Supported: T in [1, 1024], D in {64, 128}. No workspace.
 * ---------------------------------------------------------------------- */
ts_status ts_accept_commit(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok,
                           uint32_t rand_u32, int T, void* k_cache, void* v_cache, int64_t cache_stride,
                           int64_t L, const void* k_draft, const void* v_draft, int Hkv, int D,
                           ts_dtype dtype, int32_t* n_accepted, int32_t* path, int32_t* bonus,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Target-token sampling with the windowed contextual penalty (model card CLI
 * example: min-p, temperature, a penalty over a window of recent tokens; the
 * summary page's "Approach" and ablation table: penalty theta over the last W
 * tokens). Produces the target tokens that ts_accept_commit checks drafts
 * against.
 *
 *   logits     [R][V] fp32 or bf16 (dtype), R = T + 1: row 0 for the position
 *              after the committed context, row t+1 for the position after
 *              draft t. Values may be -inf, not NaN or +inf; every row needs
 *              one finite value.
 *   hist       int32 [n_hist] on the device: the most recent committed tokens,
 *              oldest first (only the last `window` are read); NULL iff n_hist = 0
 *   parent, draft_tok  int32 [T] on the device, the draft forest (entries of
 *              parent outside [-1, t) count as roots); NULL iff T = 0
 *   window     W >= 0. Row r's window is the last W tokens of hist followed,
 *              for r > 0, by the draft tokens on the root path of draft r-1.
 *              Window ids outside [0, V) are ignored.
 *   penalty    theta > 0: a windowed token's logit x becomes x / theta if
 *              x > 0, else x * theta (once per token, however often it recurs)
 *   temperature  tau >= 0; 0 = greedy: the lowest id with the largest
 *              penalised logit
 *   min_p      in [0, 1]: token i is kept when p_i >= min_p * max p, where
 *              p = softmax(penalised / tau); 0 keeps every token
 *   top_p      in (0, 1]: token i is also required to have less than top_p
 *              of the probability p on tokens strictly more probable than
 *              itself (the nucleus; tokens of equal probability are kept or
 *              dropped together); 1 keeps every token. Both filters use the
 *              same p, so the kept set is their intersection (the summary
 *              page's temperature ablation samples with top-p)
 *   u          fp32 [R] on the device, uniforms in [0, 1) drawn by the caller
 *              (may be NULL when tau = 0)
 *   tok        int32 [R] out: the smallest kept id whose cumulative kept
 *              probability (id order) exceeds u[r]; when rounding leaves
 *              u[r] at or past the end, the last kept id
 * Supported: V in [1, 1048576], T in [0, 1024]. Workspace: at least
 * ts_sample_workspace(R, V) bytes (532 bytes per row and 1024 logits, plus
 * 65,668 per row: the top-p lists), 256-byte aligned, contents ignored on
 * entry. Calls that share a workspace must not overlap.
 * ---------------------------------------------------------------------- */
size_t ts_sample_workspace(int R, int V);   /* 0 on bad sizes */

ts_status ts_sample_tokens(const void* logits, int R, int V, const int32_t* hist, int n_hist,
                           const int32_t* parent, const int32_t* draft_tok, int T, int window,
                           float penalty, float temperature, float min_p, float top_p, const float* u,
                           int32_t* tok, ts_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * 4-gram table of the committed text and top-k retrieval (tool listing, "How
 * it works": top-k candidate 4-grams become draft tokens and the n-gram table
 * is updated after verification; model card CLI example: top-k 20).
 *
 * The table is one device buffer of ts_ngram_table_bytes(capacity_log2,
 * max_entries) bytes, 256-byte aligned, owned by the caller and set up by
 * ts_ngram_init. It begins with a ts_ngram_header (copy it back to inspect):
 * min(n_entries, max_entries) distinct 4-grams are stored, and `dropped`
 * counts 4-grams that found no room (then retrieval misses them).
 * Supported: capacity_log2 in [4, 24], max_entries in [1, 262144] and at most
 * the capacity (keep the capacity at least twice the distinct 4-grams).
 *
 * ts_ngram_update: adds the 4-grams tokens[p-3 .. p] for p in [from, to), p >= 3,
 * each with its count and the last p it ended at. `tokens` is the committed
 * text on the device (int32, at least `to` entries): after a verification,
 * append the accepted drafts and the bonus token and call with the old and new
 * lengths. 0 <= from <= to <= 2^31 - 1.
 *
 * ts_ngram_retrieve: the 4-grams whose first token is *first_tok (a device
 * int32, e.g. the root of the candidate tree), ranked by count then by last
 * position, both descending; the best k (k in [1, 64]) go to out_tok [k][4]
 * (rows past the matches are -1), their counts to out_count [k] (nullable, 0
 * past the matches) and how many there are to *n_found (nullable). max_entries
 * must be the table's. Workspace: ts_ngram_retrieve_workspace(max_entries, k)
 * bytes, 256-byte aligned.
 * Calls on one table must not overlap (order them on one stream).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t capacity_log2;
  int32_t max_entries;
  int32_t n_entries;
  int32_t dropped;
} ts_ngram_header;

size_t ts_ngram_table_bytes(int capacity_log2, int max_entries);   /* 0 if unsupported */
ts_status ts_ngram_init(void* table, size_t table_bytes, int capacity_log2, int max_entries, hipStream_t stream);
ts_status ts_ngram_update(void* table, const int32_t* tokens, int64_t from, int64_t to, hipStream_t stream);
size_t ts_ngram_retrieve_workspace(int max_entries, int k);        /* 0 if unsupported */
ts_status ts_ngram_retrieve(const void* table, int max_entries, const int32_t* first_tok, int k,
                            int32_t* out_tok, int32_t* out_count, int32_t* n_found, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TS_H_ */
