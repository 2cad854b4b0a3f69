/*
 * msa.h -- C ABI of the MiniMax Sparse Attention (MSA) forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (notation of the pages):
 *   N tokens, H_q query heads, H_kv key/value heads, G = H_q / H_kv query heads
 *   per GQA group (adjacent heads: head h belongs to group r = h / G), head
 *   dimension d_h, index head dimension d_idx, key blocks of B_k tokens,
 *   k selected blocks per (query, group).
 *   - Index branch: for query i and group r, block b < L = floor(i / B_k) scores
 *     max_{j in block b} Q^idx[i, r] . K^idx[j]; the k - 1 best blocks are kept
 *     together with the local block L ("MiniMax Sparse Attention (MSA)",
 *     Deep Dive > Index Branch Architecture; Training Stability Mechanisms).
 *   - Main branch: each query head attends, with exact softmax, to the causally
 *     visible tokens of the selected blocks of its group, using the group's
 *     K/V head ("MiniMax Sparse Attention", sec. 2.1-2.2).
 *   - Execution: the selection is inverted into per-(group, block) query lists,
 *     each selected K/V block is loaded once and attended by all queries that
 *     picked it (KV-outer), one partial output per (query, block) is written,
 *     and a combine step merges the partials by log-sum-exp ("MiniMax Sparse
 *     Attention", sec. 4.2; "MiniMax Sparse Attention (MSA)", Deep Dive >
 *     KV-Outer Sparse Attention; "Optimizing MiniMax M3 Sparse Attention on
 *     NVIDIA Blackwell", sec. 1).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises, except msa_invert_status, which
 *     synchronises the given stream.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued asynchronously on it.
 *   - Every call validates its arguments on the host first.  On any error it
 *     returns a nonzero status, enqueues nothing and writes nothing.  No call
 *     throws or aborts across the ABI.
 *   - All device pointers must be 16-byte aligned (MSA_ERR_ALIGN otherwise).
 *   - bf16 is bfloat16 (upper half of IEEE binary32); fp8 is OCP FP8 E4M3
 *     ("e4m3fn", max 448).
 *   - Query rows are processed in a range [q_begin, q_begin + q_count); the
 *     keys visible to that range are [0, q_begin + q_count).  q_begin must be
 *     a multiple of B_k.  B_c = ceil((q_begin + q_count) / B_k) is the number
 *     of key blocks of the range.
 *
 * Supported shapes (MSA_ERR_UNSUPPORTED otherwise): d_h = 128, B_k in {32, 64, 128}
 * (128 for fp8 Q/K/V), d_idx in {64, 128}, G in {1, 2, 4, 8, 16}, 1 <= k <= 32,
 * B_c <= 16384 (N <= 16384 B_k), batch * H_sel * q_count * k < 2^31.
 *
 * Selection groups: H_sel = dims->H_idx when nonzero, else H_kv, index (proxy)
 * query heads, each choosing blocks for its G_sel = H_q / H_sel adjacent query
 * heads; group r reads K/V head r / (H_sel / H_kv).  Every selection-indexed
 * array below is laid out over H_sel groups of G_sel heads (with H_idx = 0
 * these are the H_kv GQA groups of G heads).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 4

enum msa_status_code {
    MSA_OK = 0,
    MSA_ERR_NULL = 1,        /* a required pointer is NULL */
    MSA_ERR_SHAPE = 2,       /* inconsistent sizes (e.g. H_q != G * H_kv) or range */
    MSA_ERR_UNSUPPORTED = 3, /* valid but outside the supported shapes above */
    MSA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
    MSA_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returned */
    MSA_ERR_HIP = 6,         /* a HIP runtime call failed (see msa_last_hip_error) */
    MSA_ERR_SCRATCH = 7      /* msa_decode_static: the step needs more scratch than
                                MSA_STATIC_SCRATCH_BYTES */
};

enum msa_dtype_code {
    MSA_DTYPE_BF16 = 0,
    MSA_DTYPE_FP8_E4M3 = 1
};

/* Problem sizes, in the pages' notation. */
typedef struct msa_dims {
    int32_t batch; /* independent sequences */
    int32_t H_q;   /* query heads */
    int32_t H_kv;  /* key/value heads = GQA groups (= index heads when H_idx = 0) */
    int32_t G;     /* query heads per group; must equal H_q / H_kv */
    int32_t d_h;   /* head dimension of Q, K, V */
    int32_t d_idx; /* head dimension of Q^idx, K^idx */
    int32_t B_k;   /* tokens per key block */
    int32_t k;     /* blocks selected per (query, group), local block included */
    int64_t N;     /* sequence length (queries = keys) */
    int32_t H_idx; /* index (proxy) query heads, each selecting blocks for its
                      H_q / H_idx adjacent query heads ("Flash-MSA", What's
                      next, note on proxy heads >= KV heads); a multiple of
                      H_kv dividing H_q, H_q / H_idx in {1, 2, 4, 8, 16};
                      0 = H_kv (one index head per GQA group) */
} msa_dims;

/* Options of the main branch. */
typedef struct msa_opts {
    int32_t qkv_dtype;   /* MSA_DTYPE_BF16 or MSA_DTYPE_FP8_E4M3 for Q, K, V */
    float softmax_scale; /* <= 0 selects 1 / sqrt(d_h) */
    float q_scale;       /* fp8 only: real value = code * scale; ignored for bf16 */
    float k_scale;
    float v_scale;
    int32_t reserved;    /* must be 0 */
    int64_t q_chunk;     /* query rows per pass of msa_forward and msa_backward:
                            a positive multiple of B_k, or 0 for the default
                            (msa_forward: MSA_DEFAULT_Q_CHUNK rows, all N when
                            N is at most that; msa_backward: all N rows) */
} msa_opts;

/* The forward's default rows per pass.  At H_q = 64 and d_h = 128 the Q rows
 * of 16,384 queries take 256 MiB, the size of MI355X's last-level (Infinity)
 * cache, so the attention's repeated Q gathers within a pass mostly hit it;
 * the per-pass selection, inversion and partial outputs also shrink to a
 * pass's rows (at N = 131,072, H_q = 64, k = 16: 4.1 GiB of workspace
 * instead of 32.6 GiB). */
#define MSA_DEFAULT_Q_CHUNK 16384

/* Library identity and diagnostics. */
int msa_abi_version(void);
const char *msa_status_string(int status);
/* hipError_t of the last failed HIP call on this thread (0 if none). */
int msa_last_hip_error(void);

/*
 * msa_index_topk -- index branch: block scores, causal block max-pool and
 * top-k with the forced local block.
 * ("MiniMax Sparse Attention (MSA)", Deep Dive > Index Branch Architecture and
 *  Exp-Free TopK Kernel; "Flash-MSA", Forward > Proxy attention.)
 *
 *   q_idx      bf16 [batch][N][H_sel][d_idx]  index queries (one head per group)
 *   k_idx      bf16 [batch][N][d_idx]         the single shared index key head
 *   block_idx  int32 [batch][H_sel][q_count][k] output: row i - q_begin of group r
 *              lists the selected block ids in ascending order, padded with -1.
 *              The local block L = floor(i / B_k) is always present and is the
 *              last valid entry; when L < k all blocks 0..L are selected.
 * Selection is on the unscaled fp32 dot products (the 1/sqrt(d_idx) factor
 * does not change the order); equal scores rank the smaller block id first.
 */
int msa_index_topk(const msa_dims *dims, const void *q_idx, const void *k_idx,
                   int64_t q_begin, int64_t q_count, int32_t *block_idx, void *stream);

/*
 * msa_index_topk_forced -- msa_index_topk with the early-training forced
 * blocks ("MiniMax Sparse Attention", ablation of the forced first block and
 * fixed local window): block 0 when force_first = 1, and the local_window - 1
 * blocks before the local block, always take slots (their scores count as
 * +inf); the remaining slots go to the best other blocks.  local_window = 1
 * and force_first = 0 is msa_index_topk.  The forced blocks must fit:
 * force_first + local_window - 1 <= k - 1 (MSA_ERR_SHAPE otherwise).
 */
int msa_index_topk_forced(const msa_dims *dims, const void *q_idx, const void *k_idx,
                          int64_t q_begin, int64_t q_count, int force_first, int local_window,
                          int32_t *block_idx, void *stream);

/*
 * msa_window_select -- the FLOP-matched sliding-window selection ("MiniMax
 * Sparse Attention", comparison with a fixed sparse pattern): query i takes
 * block 0 and the k - 1 blocks ending at its local block L = floor(i / B_k)
 * (every block 0 .. L when L < k), with no index branch.  block_idx as for
 * msa_index_topk; feed it to msa_invert_blocks, msa_sparse_attn_fwd and
 * msa_combine like a top-k selection.
 */
int msa_window_select(const msa_dims *dims, int64_t q_begin, int64_t q_count, int32_t *block_idx,
                      void *stream);

/*
 * msa_invert_workspace_size -- bytes of the device scratch buffer `sched` used by
 * msa_invert_blocks and read by msa_sparse_attn_fwd for the same range.
 */
int msa_invert_workspace_size(const msa_dims *dims, int64_t q_begin, int64_t q_count,
                              size_t *bytes);

/*
 * msa_invert_blocks -- invert the selection B[batch, group, query, slot] -> block
 * into B*[batch, group, block] -> queries, and build the pre-scheduled work
 * list of the KV-outer attention ("Flash-MSA", Backward; "MiniMax Sparse
 * Attention (MSA)", Deep Dive > KV-Outer Sparse Attention, steps 1 and 5).
 *
 *   block_idx    int32 [batch][H_sel][q_count][k] as written by msa_index_topk
 *                (any valid selection: ids in [0, floor(i / B_k)], no repeats
 *                within a row, -1 for empty slots).
 *   blk_offsets  int32 [batch][H_sel][B_c + 1] output: bin (bh, b) owns entries
 *                [blk_offsets[bh][b], blk_offsets[bh][b + 1]); the offsets are
 *                absolute positions in blk_entries (bins are laid out in
 *                (bh, b) order, so blk_offsets[bh][B_c] == blk_offsets[bh+1][0]).
 *   blk_entries  int32 [batch * H_sel * q_count * k] output (capacity): entry
 *                value (i - q_begin) * k + slot, ascending in i within a bin.
 *   sched        device scratch of msa_invert_workspace_size bytes; on return it
 *                holds the work list for msa_sparse_attn_fwd.
 * Ids outside [0, floor(i / B_k)] are skipped and counted (msa_invert_status).
 */
int msa_invert_blocks(const msa_dims *dims, const int32_t *block_idx, int64_t q_begin,
                      int64_t q_count, int32_t *blk_offsets, int32_t *blk_entries, void *sched,
                      size_t sched_bytes, void *stream);

/*
 * msa_invert_status -- synchronises `stream`, then reports how many block ids
 * the last msa_invert_blocks call on `sched` skipped as out of range.
 */
int msa_invert_status(const void *sched, int32_t *bad_ids, void *stream);

/*
 * msa_sparse_attn_fwd -- KV-outer block-sparse attention: for every (group,
 * selected block), the K/V block is staged once and every query that selected
 * it is attended with exact softmax over the block's causally visible tokens.
 * ("MiniMax Sparse Attention", sec. 4.2; "MiniMax Sparse Attention (MSA)",
 *  Deep Dive > KV-Outer Sparse Attention, steps 2-6.)
 *
 *   q         [batch][N][H_q][d_h]   bf16 or fp8 codes (opts->qkv_dtype)
 *   k, v      [batch][N][H_kv][d_h]  same dtype
 *   blk_offsets, blk_entries, sched  as produced by msa_invert_blocks for the
 *             same (q_begin, q_count)
 *   o_part    bf16 [batch][H_sel][q_count][k][G_sel][d_h] output: per (query, slot,
 *             head) the block's normalised partial output
 *             sum_j softmax_j V[j] over the block's visible tokens j
 *   lse_part  fp32 [batch][H_sel][q_count][k][G_sel] output: natural-log
 *             log-sum-exp of the scaled scores over the same tokens
 * Only slots that hold a block are written.
 */
int msa_sparse_attn_fwd(const msa_dims *dims, const msa_opts *opts, const void *q,
                        const void *k, const void *v, const int32_t *blk_offsets,
                        const int32_t *blk_entries, const void *sched, int64_t q_begin,
                        int64_t q_count, void *o_part, float *lse_part, void *stream);

/*
 * msa_combine -- split-K log-sum-exp merge of the partials of each query
 * ("MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer Sparse Attention,
 *  step 6): LSE = ln sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) * Obar_s over
 *  the valid slots s of each row: those whose block_idx entry b satisfies
 *  0 <= b <= floor(i / B_k), the test msa_invert_blocks applies.  Other
 *  slots (-1 padding, out-of-range ids) are never read, so their o_part and
 *  lse_part contents do not matter.  A row with no valid slot gets O = 0 and
 *  LSE = -inf.
 *
 *   block_idx  int32 [batch][H_sel][q_count][k]
 *   o_part, lse_part  as written by msa_sparse_attn_fwd
 *   o          bf16 [batch][N][H_q][d_h] output, rows [q_begin, q_begin + q_count)
 *   lse        fp32 [batch][N][H_q] output (may be NULL): the main-branch LSE
 */
int msa_combine(const msa_dims *dims, const int32_t *block_idx, const void *o_part,
                const float *lse_part, int64_t q_begin, int64_t q_count, void *o, float *lse,
                void *stream);

/*
 * msa_workspace_size / msa_forward -- the whole forward pass: for each chunk of
 * opts->q_chunk query rows (MSA_DEFAULT_Q_CHUNK when 0): index_topk, invert_blocks,
 * sparse_attn_fwd, combine (with several chunks, index_topk runs once over
 * all rows first).  The workspace (device memory, at least msa_workspace_size
 * bytes, 256-byte aligned) holds the per-chunk selection, inverted index,
 * work list and partial outputs, and with several chunks the whole selection.
 *
 *   q, k, v        as for msa_sparse_attn_fwd
 *   q_idx, k_idx   as for msa_index_topk
 *   o, lse         as for msa_combine (all N rows); lse may be NULL
 *   block_idx_out  int32 [batch][H_sel][N][k] (may be NULL): the selection
 */
int msa_workspace_size(const msa_dims *dims, const msa_opts *opts, size_t *bytes);
int msa_forward(const msa_dims *dims, const msa_opts *opts, const void *q, const void *k,
                const void *v, const void *q_idx, const void *k_idx, void *o, float *lse,
                int32_t *block_idx_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * msa_dense_attn_fwd -- dense causal GQA attention, the baseline MSA is
 * measured against: every query head attends, with exact softmax, to all
 * tokens j <= i of its group's K/V head ("MiniMax Sparse Attention", sec. 2.1;
 * the pages compare MSA's prefill speed with this dense form).
 *
 *   q     bf16 [batch][N][H_q][d_h]
 *   k, v  bf16 [batch][N][H_kv][d_h]
 *   o     bf16 [batch][N][H_q][d_h] output, rows [q_begin, q_begin + q_count)
 *         (other rows untouched)
 *   lse   fp32 [batch][N][H_q] output (may be NULL): natural-log log-sum-exp
 *         of the scaled scores of each row
 * Uses dims->batch, N, H_q, H_kv, G and d_h (d_idx, B_k, k and H_idx are ignored)
 * and opts->softmax_scale; q_begin needs no alignment.  Only bf16 is
 * supported (MSA_ERR_UNSUPPORTED for fp8), and batch * H_kv <= 2^20.
 */
int msa_dense_attn_fwd(const msa_dims *dims, const msa_opts *opts, const void *q,
                       const void *k, const void *v, int64_t q_begin, int64_t q_count,
                       void *o, float *lse, void *stream);

/*
 * msa_decode_workspace_size / msa_decode -- one decode step: the last token
 * of each of `batch` sequences attends to its cached tokens.  Index branch,
 * top-k with the forced local block, and the main branch over the selected
 * blocks, exactly as msa_forward computes a sequence's last row
 * ("MiniMax Sparse Attention (MSA)", Deep Dive > Index Branch Architecture,
 * Exp-Free TopK Kernel, KV-Outer Sparse Attention step 6 for the merge;
 * "MiniMax Sparse Attention", sec. 2.1-2.2; the decode-shaped query-outer
 * tile: "Optimizing MiniMax M3 Sparse Attention on NVIDIA Blackwell", sec. 1).
 *
 *   q              bf16 [batch][H_q][d_h]      the new token's queries
 *   q_idx          bf16 [batch][H_sel][d_idx]  its index queries
 *   k, v           bf16 [batch][N][H_kv][d_h]  the cache, the new token included
 *   k_idx          bf16 [batch][N][d_idx]      the index-key cache
 *   seq_lens       int32 [batch] device array (may be NULL): tokens of each
 *                  sequence, its new token at position seq_lens[b] - 1 of the
 *                  N cache slots (values are clamped to [1, N]); NULL means
 *                  every sequence has N tokens (4-byte aligned)
 *   o              bf16 [batch][H_q][d_h] output
 *   lse            fp32 [batch][H_q] output (may be NULL): natural-log LSE
 *   block_idx_out  int32 [batch][H_sel][k] (may be NULL): the selection, as a
 *                  row of msa_index_topk's output
 *   workspace      device memory of msa_decode_workspace_size bytes,
 *                  256-byte aligned: block scores, partial outputs
 * bf16 Q/K/V only (MSA_ERR_UNSUPPORTED for fp8); H_sel <= 32, batch <= 65535;
 * opts->q_chunk is ignored.
 */
int msa_decode_workspace_size(const msa_dims *dims, const msa_opts *opts, size_t *bytes);
int msa_decode(const msa_dims *dims, const msa_opts *opts, const void *q, const void *q_idx,
               const void *k, const void *v, const void *k_idx, const int32_t *seq_lens, void *o,
               float *lse, int32_t *block_idx_out, void *workspace, size_t ws_bytes, void *stream);

/*
 * msa_decode_static -- msa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same step, the same kernels and results, with the
 * workspace taken from a scratch array of MSA_STATIC_SCRATCH_BYTES that the
 * library holds in device memory, one per GPU, for the life of the process.
 * The call allocates nothing; the caller still passes every input and output.
 *
 *   arguments  as for msa_decode, without workspace and ws_bytes
 * Returns MSA_ERR_SCRATCH, before anything is enqueued, when
 * msa_decode_workspace_size exceeds MSA_STATIC_SCRATCH_BYTES (with H_sel 4,
 * k 16, G_sel 16 a step fits up to batch 237 at N = 128K, 168 at N = 1M).
 * The first call on a device looks the array's address up (with that device
 * current).  All calls on one GPU share its array: calls that may overlap on
 * one GPU (other streams, other host threads) race and must be serialised by
 * the caller; calls on one stream are ordered and safe.
 */
#define MSA_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)
int msa_decode_static(const msa_dims *dims, const msa_opts *opts, const void *q, const void *q_idx,
                      const void *k, const void *v, const void *k_idx, const int32_t *seq_lens,
                      void *o, float *lse, int32_t *block_idx_out, void *stream);

/*
 * msa_backward_workspace_size / msa_backward -- the training backward pass:
 * gradients of the sparse main attention with respect to Q, K, V ("MiniMax
 * Sparse Attention", sec. 2.2: exact softmax attention over the selected
 * tokens, differentiated), and the KL alignment gradient of the index branch
 * with respect to Q^idx and K^idx ("MiniMax Sparse Attention (MSA)", Deep
 * Dive > KL Alignment Loss; "Flash-MSA", KL Divergence Loss): for query i and
 * group r, teacher P = the mean over the group's G_sel heads of their softmax
 * over the visible selected tokens (held constant), proxy p_idx = softmax of
 * z_j = Q^idx_i,r . K^idx_j / sqrt(d_idx) over the same tokens, per-row loss
 * KL(P || p_idx), and gradient kl_weight * (p_idx - P) on z.  The selection
 * is the forward's (a constant); the work is scheduled by its inversion
 * ("Flash-MSA", Backward).
 *
 *   q, k, v, q_idx, k_idx  the forward's inputs (bf16, layouts as msa_forward)
 *   o          bf16 [batch][N][H_q][d_h]  the forward's output
 *   lse        fp32 [batch][N][H_q]       the forward's natural-log LSE
 *   d_o        bf16 [batch][N][H_q][d_h]  gradient of the loss w.r.t. o
 *   block_idx  int32 [batch][H_sel][N][k] the forward's selection
 *              (msa_forward's block_idx_out)
 *   kl_weight  multiplier of the KL gradient (e.g. the loss coefficient
 *              times 1 / (N * H_sel) for the mean over rows and groups)
 *   dq         bf16 [batch][N][H_q][d_h]   output
 *   dk, dv     bf16 [batch][N][H_kv][d_h]  output
 *   dq_idx     bf16 [batch][N][H_sel][d_idx] output    } NULL together
 *   dk_idx     bf16 [batch][N][d_idx] output            } with kl: the index
 *   kl         fp32 [batch][H_sel][N] output (may be NULL): } branch is skipped
 *              per-row KL(P || p_idx), not weighted
 *   workspace  device memory of msa_backward_workspace_size bytes, 256-byte
 *              aligned: fp32 gradient accumulators, the inversion, per-slot
 *              partials (dQ and dq_idx are sums over a row's slots) and the
 *              teacher rows the main branch hands to the index branch
 * bf16 only and B_k = 128 (MSA_ERR_UNSUPPORTED otherwise); opts->q_chunk
 * splits the query rows into chunks as in msa_forward (dK, dV and dk_idx
 * accumulate over all chunks).  Softmax scale: opts->softmax_scale (<= 0:
 * 1 / sqrt(d_h)).  fp32 atomics order the accumulation of dK, dV and dk_idx,
 * so those outputs may differ in the last bits between runs.
 */
int msa_backward_workspace_size(const msa_dims *dims, const msa_opts *opts, size_t *bytes);
int msa_backward(const msa_dims *dims, const msa_opts *opts, float kl_weight, const void *q,
                 const void *k, const void *v, const void *q_idx, const void *k_idx, const void *o,
                 const float *lse, const void *d_o, const int32_t *block_idx, void *dq, void *dk,
                 void *dv, void *dq_idx, void *dk_idx, float *kl, void *workspace, size_t ws_bytes,
                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
