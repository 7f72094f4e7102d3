/*
 * lisfa.h - C ABI of the index-selection sparse attention layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer has three steps (named on "Large Language Model Inference
 * Acceleration in Practice", section 1.2, and "Kimi New Model Open Source:
 * Day0 Inference Adaptation and Performance Optimization on Ascend",
 * section 3):
 *   1. lightning indexer: relevance scores of the current query against every
 *      cached position, weighted over the indexer heads;
 *   2. Top-K: the K most relevant visible positions, emitted as an index list;
 *   3. sparse flash attention: softmax attention of every MLA head over only
 *      the selected rows of the latent KV cache.
 * Concrete definitions used by every entry point below, for one query row r
 * (sequence b = row_seq[r], position p = row_pos[r]):
 *   score[s] = sum_j w[r,j] * max(0, q_idx[r,j,:] . k_idx[slot(b,s),:]),  s <= p
 *   idx      = the min(K, p+1) positions with the largest scores, equal scores
 *              resolved toward the lower position, sorted ascending, padded
 *              with -1 to K entries
 *   z_k      = softmax_scale * q[r,h,:] . kv[slot(b,idx_k),:]   (all D_qk cols)
 *   out[r,h] = sum_k softmax(z)_k * kv[slot(b,idx_k), :D_latent]
 *   lse[r,h] = log(sum_k exp(z_k))   (natural log)
 *
 * Conventions
 *   - Every pointer is a DEVICE pointer unless stated otherwise; the argument
 *     structs themselves live in host memory and are read during the call only.
 *   - The caller owns every buffer, including the workspace (size it with
 *     lisfa_workspace_size).  The library never allocates or frees device
 *     memory and is safe to call from several threads; its only global state
 *     is the scratch array of li_topk_sfa_noalloc (one per GPU).
 *   - All work is enqueued on `stream` (0 = the default stream) and is
 *     asynchronous; the call returns as soon as the kernels are queued.
 *     Device faults surface at the caller's next synchronisation.
 *   - Arguments are validated before anything is launched; a failing call
 *     returns a negative status and leaves every output untouched.
 *   - Out-of-range block-table entries or positions beyond a sequence's cached
 *     extent are never dereferenced: the indexer writes NaN for such a
 *     position and the attention step treats it as not selected.
 */
#ifndef LISFA_H
#define LISFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* lisfa_stream_t; /* a hipStream_t */

/* status codes */
#define LISFA_OK                   0
#define LISFA_ERR_NULL_ARG        -1
#define LISFA_ERR_BAD_SHAPE       -2
#define LISFA_ERR_BAD_DTYPE       -3
#define LISFA_ERR_WORKSPACE       -4
#define LISFA_ERR_HIP             -5
#define LISFA_ERR_UNSUPPORTED     -6

/* element types of stored tensors */
#define LISFA_BF16      0   /* bfloat16 */
#define LISFA_FP8_E4M3  1   /* OCP e4m3 (max 448), scaled by fp32 factors */
#define LISFA_MXFP8     2   /* OCP MX block format: e4m3 elements, one E8M0 scale byte
                               (2^(e-127)) per 32 consecutive elements of a row; indexer
                               queries and keys only ("Day0 Inference Adaptation and
                               Performance Optimization for Kimi K3.1 Pro", section 4) */
#define LISFA_FP8_TILE128 3 /* e4m3 codes with one fp32 factor per tile of 128 elements of
                               each row (per token and head, tile 128: the same page,
                               section 4, and "Large Language Model Inference Acceleration
                               in Practice", section 4); MLA latent cache only */

/*
 * A cache of fixed-width rows, one per token slot ("Kimi New Model Open
 * Source ...", section 3: the indexer reads the key cache stored in pages;
 * the attention step reads the main KV cache by position).  Two layouts:
 *   paged      (block_table != NULL): slot(b, s) = block_table[b*bt_stride +
 *              s / block_size] * block_size + s % block_size;
 *   contiguous (block_table == NULL): slot(b, s) = seq_base_slot[b] + s.
 * The row of slot t starts at data + t * row_stride_bytes.
 * fp8 rows are multiplied by scale[t / scale_group_tokens] (scale_group_tokens
 * consecutive physical slots share one fp32 factor; 1 = per token).
 * mxfp8 rows (width a multiple of 32): scale points to E8M0 bytes
 * [num_slots, width / 32]; element i of slot t is code * 2^(scale[t][i/32] - 127).
 */
typedef struct {
    const void*    data;               /* [num_slots, row_stride_bytes] */
    int64_t        num_slots;          /* slots in the pool (bounds checks) */
    int32_t        dtype;              /* LISFA_BF16, LISFA_FP8_E4M3, LISFA_MXFP8 or
                                          LISFA_FP8_TILE128 */
    int32_t        row_stride_bytes;   /* multiple of 16, >= row width in bytes */
    const void*    scale;              /* fp8: fp32 [num_slots / scale_group_tokens];
                                          mxfp8: uint8 E8M0 [num_slots, width / 32];
                                          fp8 tile 128: fp32 [num_slots, ceil(width / 128)],
                                          entry j covering columns [128 j, 128 j + 128),
                                          4-byte aligned; bf16: NULL */
    int32_t        scale_group_tokens; /* fp8: >= 1 */
    int32_t        block_size;         /* paged: tokens per block (> 0) */
    const int32_t* block_table;        /* paged: [num_seqs, bt_stride], else NULL */
    int32_t        bt_stride;          /* paged: entries per sequence */
    int32_t        num_seqs;           /* sequences addressable through the cache */
    const int64_t* seq_base_slot;      /* contiguous: [num_seqs], else NULL */
} lisfa_cache;

/* Lightning indexer inputs (one query row per r). */
typedef struct {
    const void*    q;            /* [R, H_I, D_I] bf16 or e4m3 codes (same dtype as k_cache) */
    const void*    q_scale;      /* fp8: fp32 [R] (per query token) or [R, H_I];
                                    mxfp8: uint8 E8M0 [R, H_I, D_I / 32]; bf16: NULL */
    int32_t        q_scale_per_head; /* fp8: 0 = [R], 1 = [R, H_I]; otherwise ignored */
    const float*   w;            /* [R, H_I] fp32 head weights */
    lisfa_cache    k_cache;      /* rows of D_I elements */
    const int32_t* row_seq;      /* [R] sequence of each query row */
    const int32_t* row_pos;      /* [R] position of each query row (sees 0..row_pos) */
    int32_t        R;            /* query rows (0 = nothing to do) */
    int32_t        H_I;          /* indexer heads: 1..64 */
    int32_t        D_I;          /* indexer head dim: 32 or 128 */
    int32_t        rows_per_group; /* >= 1: aligned groups of this many consecutive rows
                                      share one sequence (chunked prefill); the kernel
                                      then reads each key tile once per group.  A row
                                      whose row_seq differs from its group's first row
                                      gets NaN scores. */
    int64_t        max_visible;  /* host-known upper bound of row_pos[r] + 1 */
} lisfa_indexer_args;

/* Sparse MLA attention inputs. */
typedef struct {
    const void*    q;            /* [R, H, D_latent + D_rope] bf16 */
    lisfa_cache    kv_cache;     /* rows [latent (D_latent) | rope (D_rope)] */
    const int32_t* row_seq;      /* [R] */
    int32_t        R;
    int32_t        H;            /* heads: 1..128 */
    int32_t        D_latent;     /* 512 (with D_rope 64) or 64 (with D_rope 16) */
    int32_t        D_rope;
    float          softmax_scale; /* > 0 and finite (else LISFA_ERR_BAD_SHAPE) */
} lisfa_mla_args;

/*
 * li_score - lightning indexer scores ("Large Language Model Inference
 * Acceleration in Practice", section 1.2 and section 3.1, first two steps:
 * raw relevance scores, then head-weight weighting).
 *   scores: [R, ld_scores] fp32 (device). Row r receives positions
 *           0..row_pos[r]; entries after row_pos[r] are left untouched.
 *   ld_scores >= max_visible.
 * Scores are accumulated in fp32 (products of bf16 or e4m3 values are exact
 * in fp32).  fp8: score = k_scale[slot] * sum_j (w_j * q_scale) * ReLU(q8.k8),
 * which equals the definition because the scales are positive.
 * mxfp8 (D_I = 128): the dot products run on gfx950's block-scaled MFMA, which
 * applies the query's and the key's E8M0 scale to each 32-element block; rows
 * are scored one by one (rows_per_group is a hint that mxfp8 does not use).
 */
int li_score(const lisfa_indexer_args* args, float* scores, int64_t ld_scores,
             lisfa_stream_t stream);

/*
 * topk_select - per-row Top-K over precomputed scores ("Kimi New Model Open
 * Source ...", section 3: Top-K position selection that outputs only the
 * list of selected indices).
 *   scores: [R, ld_scores] fp32; row r uses entries 0..row_pos[r] (clamped to
 *           ld_scores - 1; a negative row_pos selects nothing).
 *   idx:    [R, K] int32 out, ascending positions, -1 padded.
 *   ws:     lisfa_workspace_size(LISFA_OP_TOPK, R, ld_scores, K, 0, 0) bytes
 *           (16-byte aligned), or NULL.  The size is 0 unless ld_scores >
 *           65536 and K * ceil(ld_scores / 16384) <= 16384; such rows are then
 *           selected in two passes (slices of 16384 positions keep their own
 *           Top-K, an ordered merge picks the K best).  Otherwise, or with ws
 *           NULL, long rows take a slower single-workgroup pass.
 * Exact: the order is that of the fp32 values (-0.0 == +0.0; NaN orders above
 * +inf); equal values at the K-th place go to the lower positions.  The result
 * is deterministic and the same on every path.
 */
int topk_select(const float* scores, int64_t ld_scores, const int32_t* row_pos,
                int32_t R, int32_t K, int32_t* idx, void* ws, size_t ws_bytes,
                lisfa_stream_t stream);

/*
 * li_topk - indexer scores and Top-K in one step: the per-row list of selected
 * positions without the scores ("Kimi New Model Open Source ...", section 3:
 * one operator reads the paged key cache and outputs only the index list;
 * "Large Language Model Inference Acceleration in Practice", section 3.1:
 * weighting and Top-K on chip, the pointers handed to the sparse attention).
 *   args: as li_score (row r sees positions 0..row_pos[r], clamped to
 *         max_visible rounded up to a multiple of 64).
 *   idx:  [R, K] int32 out, ascending positions, -1 padded.
 *   ws:   lisfa_workspace_size(LISFA_OP_LI_TOPK, R, max_visible, K, 0, 0) bytes,
 *         256-byte aligned (NULL when that size is 0).
 * The result equals li_score followed by topk_select on the same inputs, bit for
 * bit.  Decode rows (rows_per_group 1) with bf16 or per-token fp8 keys
 * (D_I = 128 for fp8) and MXFP8 keys are scored and selected in one launch
 * whose scores stay on chip when a row spans at most 64 workgroups of at most
 * 16384 positions and the launch has at most 256 workgroups (or one workgroup
 * per row); other shapes score into the workspace in row chunks and select
 * from there.
 */
int li_topk(const lisfa_indexer_args* args, int32_t K, int32_t* idx, void* ws,
            size_t ws_bytes, lisfa_stream_t stream);

/*
 * li_topk_plan - how these arguments are scored and selected (host function,
 * no GPU work): the number of workgroups that score and select each row in
 * the single fused launch (>= 1; the scores never reach device memory), 0 when
 * the separate score and Top-K kernels run instead, or a negative status for
 * arguments li_topk would refuse.
 *   layer = 0: li_topk, which takes the fused launch wherever the shape allows;
 *   layer = 1: the index step of li_topk_sfa, which takes it only where it is
 *              the faster path (bf16 keys, at most 4 workgroups per row).
 */
int32_t li_topk_plan(const lisfa_indexer_args* args, int32_t K, int32_t layer);

/*
 * Context parallelism: the cached positions of a sequence are split over G
 * GPUs; each GPU scores its own positions, keeps its local Top-K with the
 * scores, the candidates of all GPUs are gathered and merged into the
 * global index list, each GPU attends over the selected rows it holds, and
 * the G partial results are merged by their log-sum-exp (the Kimi K3 decode
 * article, in Japanese, part 1 item 1: with decode context parallelism each
 * GPU attends over its own region of the KV cache and a fused kernel merges
 * the partial results; "Day0 Inference Adaptation and Performance
 * Optimization for Kimi K3.1 Pro", section 5: context parallelism splits
 * long inputs along the sequence).  The gathers between GPUs are the
 * caller's (RCCL); these entry points are one GPU's share.  Every globally
 * selected position is among its own shard's local Top-K, so the merged
 * list equals the single-GPU topk_select result on the same scores.
 *
 * topk_candidates - local Top-K of one shard with scores.
 *   scores, ld_scores, row_pos: as topk_select, over the shard's local
 *           positions (local position t = logical position t + pos_offset[r]).
 *   pos_offset: [R] int32 or NULL (0).
 *   cand_pos:   [R, K] int32 out: logical positions, ascending, -1 padded.
 *   cand_score: [R, K] fp32 out: their scores (-inf for padding).
 *   ws: lisfa_workspace_size(LISFA_OP_TOPK_CANDIDATES, R, ld_scores, K, 0, 0)
 *       bytes (needed only when ld_scores > 65536; K * ceil(ld / 16384) must
 *       then be <= 16384, else LISFA_ERR_UNSUPPORTED).
 */
int topk_candidates(const float* scores, int64_t ld_scores, const int32_t* row_pos,
                    int32_t R, int32_t K, const int32_t* pos_offset, int32_t* cand_pos,
                    float* cand_score, void* ws, size_t ws_bytes, lisfa_stream_t stream);

/*
 * topk_merge - the K best of n gathered candidates per row.
 *   cand_score, cand_pos: [R, ld_cand] (first n entries used); a negative
 *           position marks no candidate.  Positions of a row must be unique.
 *   ordered: nonzero if the valid candidates of each row come in ascending
 *           position order (the local lists of a contiguous split gathered in
 *           rank order); any order is accepted with ordered = 0 (then K <=
 *           4096).  n <= 16384.
 *   idx:    [R, K] int32 out, ascending positions, -1 padded.
 *   idx_score: [R, K] fp32 out (their scores, -inf padding) or NULL.
 * Order: larger score first, equal scores toward the lower position.
 */
int topk_merge(const float* cand_score, const int32_t* cand_pos, int64_t ld_cand,
               int32_t R, int32_t n, int32_t K, int32_t ordered, int32_t* idx,
               float* idx_score, lisfa_stream_t stream);

/*
 * sparse_mla_attn - sparse flash attention over the selected rows
 * ("Large Language Model Inference Acceleration in Practice", section 1.2
 * SFA, and section 3.1, third step: read the paged KV rows named by the
 * index pointers and run attention over them).
 *   idx:  [R, K] int32 logical positions; -1 entries are skipped.  Entries
 *         must be unique.
 *   out:  [R, H, D_latent] bf16.
 *   lse:  [R, H] fp32 natural-log normaliser, or NULL.
 *   ws:   lisfa_workspace_size(LISFA_OP_SPARSE_MLA, R, 0, K, H, D_latent) bytes.
 * A row with no valid index gets out = 0 and lse = -inf.
 * Compute: bf16 MFMA with fp32 accumulation; fp8 rows are converted to bf16
 * exactly and their fp32 factor is applied to the logits and probabilities.
 */
int sparse_mla_attn(const lisfa_mla_args* args, const int32_t* idx, int32_t K,
                    void* out, float* lse, void* ws, size_t ws_bytes,
                    lisfa_stream_t stream);

/*
 * sparse_mla_attn_partial - one shard's share of sparse attention, as fp32
 * partial results for lse_combine.
 *   args: the shard's latent cache addresses its own rows: local position t
 *         of row r's sequence is logical position range[2r] + t.
 *   idx:  [R, K] int32 logical positions (the merged list); entries outside
 *         [range[2r], range[2r+1]) are skipped.  range = NULL: idx already
 *         holds local positions.
 *   out:  [R, H, D_latent] fp32 normalised output (16-byte aligned).
 *   lse:  [R, H] fp32 natural-log normaliser (required).
 *   ws:   lisfa_workspace_size(LISFA_OP_SPARSE_MLA_PARTIAL, R, 0, K, H,
 *         D_latent) bytes, 256-byte aligned.
 * A row with no selected row in the shard gets out = 0 and lse = -inf.
 */
int sparse_mla_attn_partial(const lisfa_mla_args* args, const int32_t* idx, int32_t K,
                            const int32_t* range, float* out, float* lse,
                            void* ws, size_t ws_bytes, lisfa_stream_t stream);

/*
 * lse_combine - merge G partial attention results of the same rows:
 *   M = max_g lse_g,  a_g = exp(lse_g - M),
 *   out = sum_g a_g out_g / sum_g a_g,  lse = M + log(sum_g a_g).
 *   part_out: [G, R, H, D_v] fp32 (16-byte aligned); part_lse: [G, R, H].
 *   out: [R, H, D_v] bf16 (16-byte aligned); lse: [R, H] fp32 or NULL.
 *   D_v: 64 or 512.  Parts with lse = -inf hold no row; a head with no row
 *   in any part gets out = 0 and lse = -inf.
 */
int lse_combine(const float* part_out, const float* part_lse, int32_t G, int32_t R,
                int32_t H, int32_t D_v, void* out, float* lse, lisfa_stream_t stream);

/*
 * Zigzag partition for context-parallel prefill ("Day0 Inference Adaptation
 * and Performance Optimization for a New Model", section 5.2, and the Kimi
 * K3.1 Pro page, section 5): n rows are cut into 2G segments, segment i =
 * [floor(i n / 2G), floor((i+1) n / 2G)); GPU g takes segment g and segment
 * 2G-1-g, so each GPU pairs a short causal history with a long one.
 *
 * lisfa_zigzag_share (host function): ranges[0..4) = the two [start, end)
 *   ranges of GPU g, head segment first.
 * zigzag_restore: src holds the gathered shares (GPU 0's two segments, then
 *   GPU 1's, ...), n rows of row_bytes bytes; dst receives them in original
 *   order.  src and dst must not overlap.
 */
int lisfa_zigzag_share(int64_t n, int32_t G, int32_t g, int64_t* ranges);
int zigzag_restore(const void* src, void* dst, int64_t n, int32_t G, int64_t row_bytes,
                   lisfa_stream_t stream);

/*
 * Indexer prolog ("Day0 Inference Adaptation and Performance Optimization for
 * Kimi K3.1 Pro", section 3; "Large Language Model Inference Acceleration in
 * Practice", section 3.2; "... for a New Model", section 3.2: Q quantisation
 * and K normalisation with the cache update run on separate streams ahead of
 * the index computation).  Both start from the bf16 outputs of the indexer's
 * projections (not part of this library).  Rounding to e4m3 is round to
 * nearest even with saturation to +-448.
 *
 * indexer_q_quant - dynamic quantisation of indexer queries.
 *   q: [R, H_I, D_I] bf16 (16-byte aligned); H_I <= 64, D_I 32 or 128.
 *   dtype LISFA_FP8_E4M3: q_scale_out fp32 [R], one scale per row over all
 *         heads: s = amax / 448 (1 if amax = 0), code = e4m3(x / s) (fp32
 *         IEEE division).
 *   dtype LISFA_MXFP8: q_scale_out uint8 E8M0 [R, H_I, D_I / 32]: per block of
 *         32, shared exponent floor(log2 amax) - 8 (clamped to [-127, 127], 0
 *         for a zero block), code = e4m3(x * 2^-shared) (exact scaling).
 *   q_out: [R, H_I, D_I] uint8 e4m3 codes, 16-byte aligned.
 */
int indexer_q_quant(const void* q, int32_t R, int32_t H_I, int32_t D_I, int32_t dtype,
                    void* q_out, void* q_scale_out, lisfa_stream_t stream);

/*
 * indexer_k_store - normalise new indexer keys and write them into the key
 * cache (the cache update that runs with K normalisation).
 *   k:        [T, D_I] bf16 new keys (4-byte aligned); D_I 32 or 128.
 *   normalize: nonzero = LayerNorm over the D_I elements in fp32:
 *             y = (x - mean) / sqrt(var + eps) * gamma + beta (biased
 *             variance; gamma / beta fp32 [D_I] or NULL = 1 / 0); zero = y = x.
 *   tok_seq, tok_pos: [T] int32 sequence and position of each key; the key
 *             goes to slot(tok_seq, tok_pos) of k_cache.  A key whose slot the
 *             cache cannot address (sequence out of range, block-table entry
 *             past bt_stride or negative, slot past num_slots) is skipped.
 *   k_cache:  describes the destination; its data (and scale) arrays are
 *             written.  bf16: y rounded to nearest even.  fp8
 *             (scale_group_tokens must be 1): per key s = amax / 448 written
 *             to scale[slot], codes e4m3(y / s).  mxfp8: E8M0 scales per 32
 *             elements as in indexer_q_quant.
 * Keys of one call must go to distinct slots (otherwise the survivor is
 * unspecified).
 */
int indexer_k_store(const void* k, int32_t T, int32_t D_I, const float* gamma,
                    const float* beta, float eps, int32_t normalize,
                    const int32_t* tok_seq, const int32_t* tok_pos,
                    const lisfa_cache* k_cache, lisfa_stream_t stream);

/*
 * indexer_prolog - indexer_k_store and indexer_q_quant in one launch, with the
 * arguments and results of the two (q_dtype as indexer_q_quant's dtype; the
 * keys and the queries share D_I).  The pages run these two independent parts
 * of the prolog side by side on separate streams ("Day0 Inference Adaptation
 * and Performance Optimization for a New Model", section 3.2); here one
 * launch splits its workgroups between the query rows and the keys, which
 * overlaps them without a dependency between streams.  R or T may be 0.
 * Results are bit-identical to the two calls made one after the other.
 */
int indexer_prolog(const void* q, int32_t R, int32_t H_I, int32_t D_I, int32_t q_dtype,
                   void* q_out, void* q_scale_out, const void* k, int32_t T,
                   const float* gamma, const float* beta, float eps, int32_t normalize,
                   const int32_t* tok_seq, const int32_t* tok_pos,
                   const lisfa_cache* k_cache, lisfa_stream_t stream);

/*
 * li_topk_sfa - the whole layer in one call on one stream: scores, Top-K and
 * sparse attention ("Day0 Inference Adaptation and Performance Optimization
 * for Kimi K3.1 Pro", section 3, and "Large Language Model Inference
 * Acceleration in Practice", section 3.1: scoring, weighting and selection
 * feed the sparse attention without returning to the host).  Scores and
 * partial results live in the workspace; rows are processed in chunks so the
 * score scratch stays bounded.
 *   idx_out: [R, K] int32 or NULL (then the indices live in the workspace).
 *   ws: lisfa_workspace_size(LISFA_OP_FUSED, R, max_visible, K, H, D_latent).
 * The two argument structs must agree on R and row_seq.
 */
int li_topk_sfa(const lisfa_indexer_args* iargs, const lisfa_mla_args* margs,
                int32_t K, int32_t* idx_out, void* out, float* lse,
                void* ws, size_t ws_bytes, lisfa_stream_t stream);

/*
 * li_topk_sfa_noalloc - li_topk_sfa without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The call allocates nothing:
 * the scores, index lists and partial results live in a static device array of
 * LISFA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends.  Rows are scored in chunks small enough for the
 * array; a call whose smallest layout still does not fit returns
 * LISFA_ERR_WORKSPACE (use li_topk_sfa with a caller workspace then).  The first
 * call on a GPU looks up the array's address on that GPU (the stream's device).
 * All calls on one GPU share its array: calls that overlap in time on one GPU
 * (different streams, or threads) race and must be serialised by the caller.
 * Arguments and results otherwise as li_topk_sfa.
 */
#define LISFA_NOALLOC_SCRATCH_BYTES (64ull << 20)
int li_topk_sfa_noalloc(const lisfa_indexer_args* iargs, const lisfa_mla_args* margs,
                        int32_t K, int32_t* idx_out, void* out, float* lse,
                        lisfa_stream_t stream);

#define LISFA_OP_TOPK               0   /* max_visible argument = ld_scores */
#define LISFA_OP_SPARSE_MLA         1
#define LISFA_OP_FUSED              2
#define LISFA_OP_TOPK_CANDIDATES    3   /* max_visible argument = ld_scores */
#define LISFA_OP_SPARSE_MLA_PARTIAL 4
#define LISFA_OP_LI_TOPK            5

/* Workspace bytes an entry point needs for the given sizes (host function). */
size_t lisfa_workspace_size(int32_t op, int32_t R, int64_t max_visible, int32_t K,
                            int32_t H, int32_t D_latent);

/* Human-readable text of a status code (static storage, host function). */
const char* lisfa_status_string(int32_t status);

/* ABI self-description for bindings (host functions):
 * sizeof of each argument struct: which = 0 cache, 1 indexer args, 2 mla args. */
size_t lisfa_struct_size(int32_t which);
/* Version of this header's ABI. */
int32_t lisfa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LISFA_H */
