/*
 * dsa_indexer.h - C ABI of the gfx950 (MI355X) DSA indexer library.
 *
 * The DeepSeek-Sparse-Attention indexer scores every causal prefix token of a
 * query through a pool of H_I indexer heads and keeps the k best tokens for the
 * sparse attention that follows ("MISA: Mixture of Indexer Sparse Attention for
 * Long-Context LLM Inference", technical summary, section "problem"):
 *
 *     s(t, u) = sum_j w[t, j] * max(0, q[t, j] . k[u]),   u = 0 .. pos_t,
 *
 * with signed per-head weights w ("DoSA: Dots Sparse Attention" review,
 * sections 1 and 3: signed heads, exact top-K), no scale, bias or softmax; the
 * key cache holds one key per token shared by all heads.  Ties are broken by the
 * lower token index.  Two reduced variants are provided: MISA head routing (same
 * MISA summary, sections "method" and "hierarchical variant") and HISA block
 * filtering ("HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
 * Attention" review, sections 1 and 3), and both composed (MISA∘HISA).  The
 * sparse attention that consumes the selected indices is provided too
 * (sparse_mla_attention).
 *
 * Conventions shared by every entry point
 *  - Every pointer is a DEVICE pointer (hipMalloc'ed or equivalent) on the
 *    current HIP device; tensors are dense, row-major, in the layouts below.
 *    q, k and k_pooled must be 16-byte aligned; workspace 256-byte aligned.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates device memory and keeps no pointer after a call returns.
 *  - Calls are asynchronous on `stream` (NULL = the default stream).  Argument
 *    errors return synchronously before any launch; launch errors are reported
 *    from the launch; device faults surface at the caller's synchronisation.
 *    With the environment variable DSA_DEBUG=1 every call synchronises and
 *    reports device errors itself.
 *  - On a non-zero status nothing has been launched (argument errors) or the
 *    outputs are undefined (DSA_EHIP); dsa_last_error() gives a message.
 *  - Queries: query t belongs to sequence q_seq[t] (q_seq may be NULL: all
 *    queries on sequence 0) and sits at position q_pos[t]; its causal prefix is
 *    keys 0 .. q_pos[t] inclusive.  A query whose q_seq / q_pos is out of range
 *    (q_seq not in [0, n_seq), q_pos not in [0, l_max)) gets an all-padding row.
 *  - Outputs: out_idx [nq, top_k] int32 and out_score [nq, top_k] float32
 *    (out_score may be NULL).  Row t holds K_t = min(top_k, number of
 *    candidates) selected entries first, in unspecified order (set semantics),
 *    then top_k - K_t padding entries (-1, -inf).  Returned scores are the
 *    float32 scores the selection was made on.
 *  - Workspace contents on entry are ignored (the library clears what it needs
 *    at the start of each call); two calls that run concurrently must not share
 *    a workspace.
 *  - Supported shapes (indexer calls): head_dim 64 or 128; 1 <= n_heads <= 64;
 *    bf16 inputs use MFMA, float32 inputs (dense call only) the vector ALUs;
 *    l_max (and any candidate list a pass scores) at most 67108864 =
 *    8192 * 8192 items per query (DSA_EUNSUPPORTED beyond).  The sparse
 *    attention has its own shapes, alignment and outputs, stated with it.
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DSA_OK 0
#define DSA_EINVAL 1       /* bad shape, pointer, alignment or argument combination */
#define DSA_EUNSUPPORTED 2 /* valid but not implemented (e.g. head_dim not 64/128) */
#define DSA_EWORKSPACE 3   /* workspace_bytes smaller than the *_workspace_size value */
#define DSA_EHIP 4         /* a HIP call or kernel launch failed */
#define DSA_ETIMEOUT 5     /* (DSA_DEBUG only) a HISA query's bounded wait gave up; see out_status */

/* input element types of q, k (and k_pooled) */
#define DSA_DTYPE_BF16 0   /* bf16 carried as 16-bit patterns */
#define DSA_DTYPE_F32 1

/* Message for the last non-zero status returned on the calling thread. */
const char* dsa_last_error(void);

/* ABI version of this header (increments on any signature change). */
int dsa_abi_version(void);

/*
 * Dense DSA indexer: score every prefix key of every query with all n_heads
 * heads and select the top_k keys (MISA summary, section "problem").
 *
 *   q       [nq, n_heads, head_dim]    dtype
 *   w       [nq, n_heads]              float32, signed
 *   k       [n_seq, l_max, head_dim]   dtype   (indexer key cache)
 *   q_seq   [nq] int32 or NULL,  q_pos [nq] int32
 *   out_idx [nq, top_k] int32 token indices;  out_score [nq, top_k] or NULL
 * 1 <= top_k <= 1048576.  Workspace: indexer_score_topk_workspace_size(...).
 */
size_t indexer_score_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                         int32_t n_seq, int64_t l_max, int32_t top_k,
                                         int32_t dtype);
int indexer_score_topk(const void* q, const float* w, const void* k, int32_t dtype,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t nq, int32_t n_heads,
                       int32_t head_dim, int32_t n_seq, int64_t l_max, int32_t top_k,
                       int32_t* out_idx, float* out_score, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * The dense indexer call for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, semantics and kernels as indexer_score_topk, without the
 * workspace: it uses instead a device array of DSA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on (allocated when the library's code
 * is loaded on that GPU, kept until the process ends).  It calls no hipMalloc,
 * hipFree or other allocating routine; the first call on a device looks the
 * array's address up (hipGetSymbolAddress) with that device current.
 *  - A call whose indexer_score_topk_workspace_size exceeds
 *    DSA_NOALLOC_SCRATCH_BYTES returns DSA_EUNSUPPORTED before any launch
 *    (the dense decode workload, 64 queries x 131072 keys, needs 68,161,792).
 *  - Every call on one GPU shares that GPU's array and clears what it needs at
 *    its start: calls that overlap in time on one GPU (other streams, other
 *    host threads) race and give undefined results; serialise them.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (80u << 20)
int indexer_score_topk_noalloc(const void* q, const float* w, const void* k, int32_t dtype,
                               const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                               int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                               int32_t top_k, int32_t* out_idx, float* out_score,
                               hipStream_t stream);

/*
 * Certified exact top-k of the dense indexer (DoSA review, sections 1 and 3:
 * screen with part of the heads, bound the others, prune, rescore the
 * survivors with every head and select; the page gives no formulas, these
 * bounds are derived from Cauchy-Schwarz).  Same result as indexer_score_topk
 * on the same inputs (the rescoring scores every survivor with all heads
 * exactly as the dense call does; ties: lower index):
 *  1. screened heads S: the n_screen_heads heads of largest |w_j| * |q_j|
 *     (ties: lower j); every other head j adds w_j * max(0, q_j . k) with
 *     0 <= max(0, q_j . k) <= |q_j| |k|, so with s_S the score over S,
 *       LB = s_S + |k| * sum_{j not in S, w_j < 0} w_j |q_j|,
 *       UB = s_S + |k| * sum_{j not in S, w_j > 0} w_j |q_j|
 *     (each widened by 2^-12 (|s_S| + |k| sum_j |w_j| |q_j|) for rounding);
 *  2. tau = the top_k-th largest LB of the query (every key kept when its
 *     prefix holds fewer than top_k keys);
 *  3. survivors: the keys with UB >= tau (no other key can be selected);
 *  4. every head over the survivors, then the exact top_k.
 * The screening pass reads the whole key cache, like the dense call, and the
 * rescoring gathers the survivors' rows again: the call pays off only when few
 * keys survive (on inputs with little structure nearly every key survives).
 *
 *   out_survivors [nq] int32 survivor count of each query, or NULL
 * Only DSA_DTYPE_BF16; 1 <= n_screen_heads <= min(n_heads, 16); l_max <=
 * 65535 * 4096.  Other arguments as for indexer_score_topk.  Workspace:
 * indexer_certified_topk_workspace_size(...) (8 * nq * l_max bytes for the
 * bounds and survivor lists, plus one set of candidate segments).
 */
size_t indexer_certified_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                             int32_t n_seq, int64_t l_max,
                                             int32_t n_screen_heads, int32_t top_k);
int indexer_certified_topk(const void* q, const float* w, const void* k, int32_t dtype,
                           const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                           int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                           int32_t n_screen_heads, int32_t top_k, int32_t* out_idx,
                           float* out_score, int32_t* out_survivors, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Mean-pooled block keys (MISA summary, "method" step 1: M = ceil(L/B) blocks
 * and mean-pooled indexing keys; HISA review, section 3: pooled representative
 * vector per block of size B).  Block b of sequence s covers tokens
 * [b*block, min((b+1)*block, l_max)); its pooled key is their mean, accumulated
 * in float64 and rounded once to bf16 (round to nearest, ties to even).
 *
 *   k         [n_seq, l_max, head_dim]             bf16
 *   k_pooled  [n_seq, ceil(l_max/block), head_dim] bf16 (written)
 * Only DSA_DTYPE_BF16.  Needs no workspace.
 */
int indexer_mean_pool_keys(const void* k, int32_t dtype, int32_t n_seq, int64_t l_max,
                           int32_t head_dim, int32_t block, void* k_pooled, hipStream_t stream);

/*
 * MISA head-routed indexer (MISA summary, "method"): the router scores the
 * query's pooled block keys with all heads, importance
 *   I[t, j] = |w[t, j]| * sum_{b < M_t} max(0, q[t, j] . kbar[b]),  M_t = ceil((q_pos[t]+1)/block),
 * keeps the n_active_heads (h) most important heads (ties: lower head index),
 * and only those heads score every prefix token with their original weights.
 *  - k_prime == 0 (MISA): out_idx / out_score = top_k of the h-head scores.
 *  - k_prime >= top_k (MISA dagger, "hierarchical variant"): the h-head pass
 *    keeps k_prime candidates (written to out_cand [nq, k_prime] if not NULL,
 *    padded with -1), all heads rescore them, and out_idx / out_score are the
 *    top_k of the full scores.
 * The pooled keys of a query's partial last block (when (q_pos+1) % block != 0)
 * are computed from k, so k_pooled only needs to hold full blocks.
 *
 *   k_pooled  [n_seq, ceil(l_max/block), head_dim] bf16 from
 *             indexer_mean_pool_keys, or NULL (then the call pools into its
 *             workspace first, which reads the whole key cache)
 *   out_heads [nq, h] int32 routed heads, most important first, or NULL
 *   out_importance [nq, n_heads] float32 router importance, or NULL
 * Only DSA_DTYPE_BF16; 1 <= h <= n_heads; 1 <= block.
 */
size_t misa_route_score_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                            int32_t n_seq, int64_t l_max, int32_t block,
                                            int32_t n_active_heads, int32_t k_prime,
                                            int32_t top_k, int32_t pooled_given);
int misa_route_score_topk(const void* q, const float* w, const void* k, const void* k_pooled,
                          int32_t dtype, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                          int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                          int32_t block, int32_t n_active_heads, int32_t k_prime, int32_t top_k,
                          int32_t* out_idx, float* out_score, int32_t* out_heads,
                          float* out_importance, int32_t* out_cand, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * HISA block-filtered indexer (HISA review, sections 1 and 3): block scores
 *   bs[t, b] = sum_j w[t, j] * max(0, q[t, j] . kbar[b]),  b < M_t,
 * keep the m_blocks best blocks (ties: lower block index), then score the
 * tokens of the surviving blocks (clipped to the prefix) with all heads and
 * keep the top_k.  Partial last blocks are pooled from k as for MISA.
 *
 *   out_blocks [nq, m_blocks] int32 surviving blocks (padded with -1) or NULL
 *   out_block_score [nq, m_blocks] float32 their block scores, or NULL
 *   out_status [nq] int32 or NULL (4-byte aligned): 0 when the query's row is
 *             complete, 1 when the token pass of that query gave up its
 *             bounded wait for the query's block selection (about 0.67 s; see
 *             dsa_hisa_wait_limit) - that row of out_idx / out_score then
 *             holds padding only (-1, -inf), never a partial selection; the
 *             kept blocks are still reported.  With DSA_DEBUG=1 the call also
 *             returns DSA_ETIMEOUT when any query timed out.
 * Only DSA_DTYPE_BF16; 1 <= m_blocks; 1 <= block.
 */
size_t hisa_block_filter_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                             int32_t n_seq, int64_t l_max, int32_t block,
                                             int32_t m_blocks, int32_t top_k,
                                             int32_t pooled_given);
int hisa_block_filter_topk(const void* q, const float* w, const void* k, const void* k_pooled,
                           int32_t dtype, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                           int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max,
                           int32_t block, int32_t m_blocks, int32_t top_k, int32_t* out_idx,
                           float* out_score, int32_t* out_blocks, float* out_block_score,
                           int32_t* out_status, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * MISA then HISA (MISA summary, "method": the head axis; HISA review,
 * section 3: the token axis; the composition, which the pages name but do
 * not spell out, routes first): the n_active_heads = h most important heads
 * of every query are chosen by MISA's router (importance as for
 * misa_route_score_topk), and both HISA stages use only them, original
 * weights kept: block scores
 *   bs[t, b] = sum_{j in heads_t} w[t, j] * max(0, q[t, j] . kbar[b]),
 * the m_blocks best blocks, then token scores with the same heads inside the
 * surviving blocks and the top_k.  Outputs as for hisa_block_filter_topk
 * (out_status included), plus out_heads [nq, h] (most important first) and
 * out_importance [nq, n_heads], each optional.
 * Only DSA_DTYPE_BF16; 1 <= h <= n_heads; 1 <= block; 1 <= m_blocks <= 1024,
 * m_blocks * block <= 8192 and ceil(l_max / block) <= 131072
 * (DSA_EUNSUPPORTED otherwise); nq <= 65535.
 */
size_t misa_hisa_topk_workspace_size(int32_t nq, int32_t n_heads, int32_t head_dim,
                                     int32_t n_seq, int64_t l_max, int32_t block,
                                     int32_t n_active_heads, int32_t m_blocks, int32_t top_k,
                                     int32_t pooled_given);
int misa_hisa_topk(const void* q, const float* w, const void* k, const void* k_pooled,
                   int32_t dtype, const int32_t* q_seq, const int32_t* q_pos, int32_t nq,
                   int32_t n_heads, int32_t head_dim, int32_t n_seq, int64_t l_max, int32_t block,
                   int32_t n_active_heads, int32_t m_blocks, int32_t top_k, int32_t* out_idx,
                   float* out_score, int32_t* out_heads, float* out_importance,
                   int32_t* out_blocks, float* out_block_score, int32_t* out_status,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bound of the HISA token pass's wait for its query's block selection, in
 * ticks of the GPU's 100 MHz wall clock, for the calls that start after this
 * one (process-wide).  ticks < 0 restores the default (2^26, about 0.67 s);
 * 0 makes a wait give up at its first unsuccessful check, which lets a test
 * drive the timeout path with every kernel still ending normally.  The wait
 * only ends early when other work holds the compute units that the query's
 * block selection needs.  Returns DSA_OK.
 */
int dsa_hisa_wait_limit(int64_t ticks);

/*
 * Sparse attention over the selected index list, the operator the indexer
 * feeds (HISA review, key terms and section 3: the selected indices go to
 * Sparse MLA unchanged; IndexCache review, section 1: O(L k) attention with
 * k selected tokens).  The pages give no formula; the reading taken is
 * scaled-softmax attention in absorbed multi-head latent attention form: one
 * latent row c[s, u] of d_qk = 576 values per token is the key of every head,
 * its first d_v = 512 values are the value, and for query t and head h
 *   o[t, h] = sum_i softmax_i(softmax_scale * q[t, h] . c[s_t, idx[t, i]])
 *             * c[s_t, idx[t, i], 0:512]
 * over the entries of idx[t] inside the prefix 0..q_pos[t] (others, such as
 * the -1 padding of the top-k outputs, are skipped; a repeated entry counts
 * each time).  A query with no valid entry, or with an invalid (seq, pos),
 * gets zeros.
 *   q [nq, n_heads, 576] bf16;  kv [n_seq, l_max, 576] bf16 latent cache;
 *   q_seq [nq] int32 or NULL (all on cache 0);  q_pos [nq] int32;
 *   idx [nq, top_k] int32 (e.g. the out_idx of an indexer call);
 *   out [nq, n_heads, 512] bf16.
 * fp32 accumulation; probabilities rounded to bf16 for the value product.
 * Only DSA_DTYPE_BF16, d_qk = 576, d_v = 512, n_heads in {32, 64, 96, 128},
 * 1 <= top_k <= 32768 (DSA_EUNSUPPORTED otherwise).  q, kv and out 16-byte
 * aligned.  The workspace holds the per-slice partial outputs when a query's
 * list is split over several workgroups (zero bytes otherwise).
 */
size_t sparse_mla_workspace_size(int32_t nq, int32_t n_heads, int32_t d_qk, int32_t d_v,
                                 int32_t top_k);
int sparse_mla_attention(const void* q, const void* kv, int32_t dtype, const int32_t* q_seq,
                         const int32_t* q_pos, const int32_t* idx, int32_t nq, int32_t n_heads,
                         int32_t d_qk, int32_t d_v, int32_t n_seq, int64_t l_max, int32_t top_k,
                         float softmax_scale, void* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Selection agreement (MISA summary, "results"; HISA review, section 3): per
 * query IoU = |A & B| / |A | B| over the non-negative entries of a[t, :] and
 * b[t, :] (two empty rows give 1).  Rows must hold no duplicate indices.
 *   a, b [nq, k] int32;  out_iou [nq] float32;  1 <= k <= 8192.
 */
int indexer_selection_iou(const int32_t* a, const int32_t* b, int32_t nq, int32_t k,
                          float* out_iou, hipStream_t stream);

/*
 * Kernel timing, for measurement.  While enabled (dsa_kernel_timing(1)), every
 * kernel the library launches is bracketed by two HIP events recorded on the
 * call's stream, tagged with its kernel kind (DSA_KERNEL_*).  Events come from
 * a pool the library creates once and reuses (hipEventCreate, no device memory).
 * dsa_kernel_timing_read() waits for the recorded events, returns for one kind
 * the number of launches and their summed / minimum / maximum duration in
 * milliseconds, and forgets the records of that kind.  Disabling drops all
 * pending records.  Not thread-safe against concurrent calls that record.
 */
#define DSA_KERNEL_PREPARE 0      /* workspace clear + partial-block pooling */
#define DSA_KERNEL_SCORE_TOKENS 1 /* score-and-emit over prefix tokens */
#define DSA_KERNEL_SCORE_POOLED 2 /* score-and-emit over pooled blocks (HISA stage 1) */
#define DSA_KERNEL_SCORE_LIST 3   /* score-and-emit over a candidate list (MISA dagger) */
#define DSA_KERNEL_SCORE_BLOCKS 4 /* score-and-emit over surviving blocks (HISA stage 2) */
#define DSA_KERNEL_ROUTE 5        /* MISA router */
#define DSA_KERNEL_POOL 6         /* mean pooling */
#define DSA_KERNEL_IOU 7
#define DSA_KERNEL_PREFILL 8      /* prefill-shaped scoring */
#define DSA_KERNEL_ROWSELECT 9    /* prefill row selection */
#define DSA_KERNEL_MERGE 10       /* exact top-k merge after a score-and-emit kernel */
#define DSA_KERNEL_ROUTE_HEADS 11 /* MISA head selection (prefill shape) */
#define DSA_KERNEL_PREFILL_ROUTED 12 /* MISA routed scoring on the prefill shape */
#define DSA_KERNEL_HISA 13        /* HISA in one kernel: blocks, top-m, tokens, top-k */
#define DSA_KERNEL_MLA 14         /* sparse attention over the index list (+ slice merge) */
#define DSA_KERNEL_CERTIFY 15     /* certified top-k: screened heads and bounds, survivor lists */
#define DSA_KERNEL_KINDS 16
int dsa_kernel_timing(int enable);
int dsa_kernel_timing_read(int32_t kind, int64_t* launches, double* total_ms, double* min_ms,
                           double* max_ms);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H */
