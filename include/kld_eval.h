/*
 * kld_eval.h -- C ABI of the MI355X (gfx950) quantized-vs-base logit comparison.
 *
 * The operation. For every token position the caller holds two rows of
 * next-token logits over the full vocabulary: one from the base (BF16) model
 * and one from the quantized model. For each row pair the library computes
 *   - the KL divergence KL(P_base || Q_quant) of the quantized model's softmax
 *     from the base model's softmax, in nats, at temperature 1, over all
 *     `vocab` entries ("Mistral-Small-4-119B-2603 GSQ-RCO IQ3_S GGUF" model card,
 *     "How it was made" step 5 and the "Quality" section; "Qwen3.6 27B
 *     Quantization Benchmark", section "Understand KLD and Same Top P");
 *   - the argmax of each row, ties broken toward the lowest index, and whether
 *     the two argmaxes agree -- the "Same Top P" / same-top-1 test (same
 *     section of the Qwen3.6 benchmark page; "Unsloth Dynamic 3.0 GGUFs",
 *     "The Divergence-300 @32 Metric", which calls top-1 an argmax on one
 *     prediction);
 * and reduces the per-token values to the mean KLD, the max KLD (with its row)
 * and the fraction of rows whose top tokens agree, over every row evaluated
 * (the "Raw benchmark data" table of the Qwen3.6 page reports exactly such
 * means). The base logits are produced once and compared against each quant
 * in turn ("Measurement method" on the same page), so rows can be fed in any
 * order and in pieces, and reduced once.
 *
 * Layout. `base` and `quant` are device pointers to row-major, contiguous
 * [n_rows, vocab] arrays; row r starts at element r * vocab. Element types are
 * IEEE float32 or bfloat16 (1 sign, 8 exponent, 7 mantissa bits), chosen per
 * tensor at create time; bfloat16 is widened exactly to float32. All logits
 * must be finite: non-finite inputs give unspecified (but memory-safe)
 * results. The fastest path needs vocab % 8 == 0 and 16-byte-aligned row
 * pointers; any other shape is still handled, more slowly.
 *
 * Ownership. The caller owns `base`, `quant` and every `*_out` array (device
 * memory). The handle owns its per-token buffers (max_rows rows), the
 * reduction partials and a pinned host summary. Nothing is retained from the
 * caller's pointers after the work enqueued by a call has run.
 *
 * Streams. `stream` is a hipStream_t passed as void*; NULL means the default
 * stream. kld_eval_rows only enqueues work. kld_eval_reduce orders itself
 * after every earlier kld_eval_rows call on this handle, whatever stream it
 * used, and blocks until the summary is on the host.
 *
 * Errors. Every call returns a kld_status. Arguments are validated on the host
 * before any work is enqueued; an invalid call enqueues and writes nothing.
 * Errors reported by HIP while enqueueing or running work are latched in the
 * handle and returned by the next kld_eval_reduce / kld_eval_destroy.
 * kld_eval_last_error() returns a message for the calling thread's last
 * non-OK status. No C++ exception crosses this interface.
 *
 * Threading. Calls on one handle may come from several threads as long as
 * concurrent kld_eval_rows calls cover disjoint row ranges (the reductions
 * share one workspace per handle and run one at a time); results are
 * deterministic: for one handle they are bit-identical whatever the chunking,
 * call order or streams (the launch shape, and so the summation order, is a
 * function of the element types and the handle's max_rows only).
 */
#ifndef KLD_EVAL_H
#define KLD_EVAL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kld_eval kld_eval; /* opaque handle */

typedef enum kld_dtype {
    KLD_DTYPE_F32 = 0,  /* IEEE binary32 */
    KLD_DTYPE_BF16 = 1  /* bfloat16, raw 16-bit patterns */
} kld_dtype;

typedef enum kld_status {
    KLD_OK = 0,
    KLD_ERR_INVALID_ARG = -1,      /* NULL pointer, vocab < 1, bad dtype, negative count ... */
    KLD_ERR_NO_DEVICE = -2,        /* no HIP device visible */
    KLD_ERR_UNSUPPORTED_ARCH = -3, /* current device is not gfx950 */
    KLD_ERR_OUT_OF_MEMORY = -4,    /* a device or pinned allocation failed */
    KLD_ERR_RANGE = -5,            /* row_offset + n_rows exceeds max_rows */
    KLD_ERR_HIP = -6,              /* HIP reported an error (latched) */
    KLD_ERR_BAD_HANDLE = -7,       /* NULL, destroyed or foreign handle */
    KLD_ERR_EMPTY = -8             /* reduce over zero rows */
} kld_status;

typedef struct kld_eval_summary {
    int64_t n_rows;      /* rows reduced */
    double kld_sum;      /* sum of per-token KLD (float64 accumulation, fixed order) */
    double kld_mean;     /* kld_sum / n_rows */
    double kld_max;      /* largest per-token KLD */
    int64_t kld_max_row; /* lowest row index attaining kld_max */
    int64_t n_match;     /* rows whose base and quant argmax agree */
    double same_top1;    /* n_match / n_rows */
} kld_eval_summary;

/*
 * Token-conditioned metrics over the rows whose next-token id t is in
 * [0, vocab). With log p(t) = z[t] - lse, per model:
 *   ppl_base = exp(-logp_base_sum / n_scored), ppl_quant likewise -- the
 *   "Mean PPL(Q)" column of the Qwen3.6 benchmark's "Raw benchmark data"
 *   table; ppl_ratio = ppl_quant / ppl_base, the perplexity ratio of the
 *   GSQ-RCO model card's "Quality" section; dp = q(t) - p(t), the change of
 *   the actual token's probability ("points" in that section), with its mean
 *   and its root mean square (the table's "RMS Δp (%)", as a fraction here).
 * A perplexity past the largest double is +inf; ppl_ratio is computed as
 * exp((logp_base_sum - logp_quant_sum) / n_scored), the same quantity, and
 * stays finite there. With n_scored == 0 every mean is NaN.
 */
typedef struct kld_eval_token_summary {
    int64_t n_scored;      /* rows with 0 <= t < vocab */
    int64_t n_invalid;     /* rows with t >= vocab: not scored, counted here */
    double logp_base_sum;  /* sum of log p_base(t) over scored rows (float64, fixed order) */
    double logp_quant_sum; /* sum of log p_quant(t) */
    double ppl_base;       /* exp(-logp_base_sum / n_scored) */
    double ppl_quant;      /* exp(-logp_quant_sum / n_scored) */
    double ppl_ratio;      /* ppl_quant / ppl_base = exp((logp_base_sum - logp_quant_sum) / n_scored) */
    double dp_mean;        /* mean of q(t) - p(t) */
    double dp_rms;         /* sqrt(mean of (q(t) - p(t))^2) */
} kld_eval_token_summary;

/*
 * Create a handle on the current HIP device for rows of `vocab` logits.
 *   vocab      1 .. 2^31-1 entries per row
 *   max_rows   >= 1: capacity of the per-token buffers (rows addressable by
 *              row_offset + r in kld_eval_rows)
 *   base_dtype, quant_dtype: a kld_dtype each
 * Returns KLD_ERR_INVALID_ARG, KLD_ERR_NO_DEVICE, KLD_ERR_UNSUPPORTED_ARCH or
 * KLD_ERR_OUT_OF_MEMORY on failure, with *out set to NULL.
 */
kld_status kld_eval_create(kld_eval** out, int64_t vocab, int64_t max_rows,
                           int32_t base_dtype, int32_t quant_dtype);

/*
 * Compare n_rows row pairs and store their per-token results at handle rows
 * [row_offset, row_offset + n_rows). Row r of `base`/`quant` is handle row
 * row_offset + r. Asynchronous on `stream`.
 *   kld_out          float32[n_rows]  KL(P_base || Q_quant) per row, nats
 *   match_out        uint8[n_rows]    1 when the argmaxes agree, else 0
 *   argmax_base_out  int32[n_rows]    lowest index of the base row's maximum
 *   argmax_quant_out int32[n_rows]    lowest index of the quant row's maximum
 * Each *_out is an optional device array (NULL skips it); the handle's own
 * buffers are always written. n_rows == 0 is a no-op. Rows whose single
 * pass's fp32 sums would lose the 1e-5 relative accuracy (one row far
 * flatter than the other, or far-apart dominant tokens) are evaluated a
 * second time in float64 by the same kernel (kld_eval_copy_row_flags reports
 * which, and why). Returns
 * KLD_ERR_RANGE when row_offset + n_rows > max_rows, KLD_ERR_INVALID_ARG for
 * NULL inputs or negative counts, KLD_ERR_HIP if the launch fails.
 */
kld_status kld_eval_rows(kld_eval* h, const void* base, const void* quant,
                         int64_t n_rows, int64_t row_offset,
                         float* kld_out, uint8_t* match_out,
                         int32_t* argmax_base_out, int32_t* argmax_quant_out,
                         void* stream);

/*
 * kld_eval_rows plus the token-conditioned metrics, in the same pass.
 *   tokens           int32[n_rows] device array: the id of the token that
 *                    follows each position. 0 <= t < vocab is scored; t < 0
 *                    marks a position with no next token (not scored); t >=
 *                    vocab is not scored and counted as invalid. NULL makes
 *                    this call identical to kld_eval_rows.
 *   logp_base_out    float32[n_rows]  log p_base(t), NaN where not scored
 *   logp_quant_out   float32[n_rows]  log p_quant(t), NaN where not scored
 *   dp_out           float32[n_rows]  p_quant(t) - p_base(t), NaN where not scored
 * Other arguments, outputs and errors as for kld_eval_rows; every *_out may be
 * NULL. Rows written by kld_eval_rows are "not scored".
 */
kld_status kld_eval_rows_tokens(kld_eval* h, const void* base, const void* quant,
                                const int32_t* tokens, int64_t n_rows, int64_t row_offset,
                                float* kld_out, uint8_t* match_out,
                                int32_t* argmax_base_out, int32_t* argmax_quant_out,
                                float* logp_base_out, float* logp_quant_out, float* dp_out,
                                void* stream);

/*
 * kld_eval_rows with its kernel timed by the launch itself, for callers that
 * measure the row pass without adding packets to the stream.
 *   start_event, stop_event  hipEvent_t (as void*), each may be NULL; created
 *                    by the caller (with timing, on the handle's device) and
 *                    still owned by it. The row kernel's dispatch records
 *                    start when the call's first launch begins and stop when
 *                    its last launch ends (hipExtLaunchKernel); the
 *                    elapsed time between them is the row pass alone. Neither
 *                    is recorded when n_rows == 0 or the call fails before
 *                    launching.
 * Results, outputs, ordering and errors as for kld_eval_rows (bit-identical
 * per-token results).
 */
kld_status kld_eval_rows_timed(kld_eval* h, const void* base, const void* quant,
                               int64_t n_rows, int64_t row_offset,
                               float* kld_out, uint8_t* match_out,
                               int32_t* argmax_base_out, int32_t* argmax_quant_out,
                               void* stream, void* start_event, void* stop_event);

/*
 * Reduce handle rows [0, n_rows) -- which must all have been written by
 * kld_eval_rows -- to a summary: float64 sum and mean of the per-token KLD,
 * the max and its lowest row, the match count and fraction. Deterministic:
 * the result depends only on the per-token values, not on how the rows were
 * chunked or which streams computed them. Blocks until *out is filled.
 * The handle keeps the results of its last reduction: a reduction (this call,
 * kld_eval_reduce_tokens or kld_eval_reduce_segments) over the same rows or
 * segments, with no kld_eval_rows* or kld_eval_rows_topk call in between,
 * returns them without launching anything.
 * Returns KLD_ERR_EMPTY for n_rows == 0, KLD_ERR_RANGE for n_rows > max_rows,
 * or a latched KLD_ERR_HIP.
 */
kld_status kld_eval_reduce(kld_eval* h, int64_t n_rows, kld_eval_summary* out, void* stream);

/*
 * kld_eval_reduce without the wait: enqueues the same reduction of handle rows
 * [0, n_rows) on `stream` and returns. The summary (the same bits
 * kld_eval_reduce returns) is written to *out, which must be memory the
 * device can write: device memory, or pinned host memory (hipHostMalloc);
 * read it once the stream has reached this point. Ordered after earlier
 * kld_eval_rows calls on any stream, and later reductions of this handle on
 * other streams order after it; rows overwritten by a later kld_eval_rows
 * call before this work runs give an undefined summary. Returns
 * KLD_ERR_INVALID_ARG for a NULL out, KLD_ERR_EMPTY for n_rows == 0,
 * KLD_ERR_RANGE for n_rows > max_rows, KLD_ERR_HIP for a latched error or a
 * failed launch.
 */
kld_status kld_eval_reduce_async(kld_eval* h, int64_t n_rows, kld_eval_summary* out, void* stream);

/*
 * Token-conditioned summary of handle rows [0, n_rows), computed by the same
 * deterministic reduction as kld_eval_reduce (float64 sums in a fixed order).
 * Blocks until *out is filled. Errors as for kld_eval_reduce.
 */
kld_status kld_eval_reduce_tokens(kld_eval* h, int64_t n_rows, kld_eval_token_summary* out, void* stream);

/*
 * Per-segment summaries: segment s covers handle rows
 * [offsets[s], offsets[s + 1]), for s in [0, n_segments) -- one summary per
 * context, per fixed-length chunk or per domain, as the pages report them
 * (GSQ-RCO model card, "Quality": per domain, over chunks of 512 tokens).
 *   offsets     host int64[n_segments + 1], non-decreasing, offsets[0] >= 0,
 *               offsets[n_segments] <= max_rows; every row in a segment must
 *               have been written. Segments may be empty and need not cover
 *               every row.
 *   kld_out     host kld_eval_summary[n_segments] (NULL skips). An empty
 *               segment has n_rows 0, NaN mean and fraction, kld_max -inf and
 *               kld_max_row -1.
 *   tok_out     host kld_eval_token_summary[n_segments] (NULL skips).
 * A segment [0, n) gives bit-for-bit what kld_eval_reduce and
 * kld_eval_reduce_tokens give for n rows. The handle grows a workspace for
 * more than one segment on first use (KLD_ERR_OUT_OF_MEMORY if that fails).
 * Blocks until the outputs are filled. Returns KLD_ERR_INVALID_ARG for NULL
 * offsets, n_segments outside [1, 2^30] or decreasing offsets, KLD_ERR_RANGE
 * for offsets outside [0, max_rows], or a latched KLD_ERR_HIP.
 */
kld_status kld_eval_reduce_segments(kld_eval* h, const int64_t* offsets, int64_t n_segments,
                                    kld_eval_summary* kld_out, kld_eval_token_summary* tok_out,
                                    void* stream);

/*
 * Copy the log-normalisers log(sum_i exp z_i) of handle rows
 * [row_offset, row_offset + n_rows), as computed by kld_eval_rows, to device
 * arrays (float32[n_rows] each, NULL skips). Asynchronous on `stream`, ordered
 * after earlier kld_eval_rows calls on any stream.
 */
kld_status kld_eval_copy_lse(kld_eval* h, int64_t row_offset, int64_t n_rows,
                             float* lse_base_out, float* lse_quant_out, void* stream);

/*
 * Conditioning flags of handle rows [row_offset, row_offset + n_rows): one
 * byte per row, written by the kld_eval_rows / kld_eval_rows_tokens call that
 * last wrote the row (0 for rows no such call has written; kld_eval_rows_topk
 * does not touch them). A nonzero byte means the row's single-pass fp32 sums
 * could not be trusted to the stated accuracy, and the same call evaluated
 * the row a second time in float64 (the KL definition of the GSQ-RCO model
 * card, "How it was made" step 5, summed term by term) and stored that
 * result. Bits:
 *   KLD_ROW_FLAG_AMPLIFIED   the sums' rounding is amplified past the KL
 *                            tolerance: one distribution far flatter than
 *                            the other
 *   KLD_ROW_FLAG_QUANT_MASS  the quant row's mass relative to its maximum is
 *                            under 1/4 of the base row's: its normaliser lost
 *                            bits to cancellation
 *   KLD_ROW_FLAG_CARRIED     rescales moved more mass between the two sums
 *                            than the quant normaliser's bound allows: one
 *                            row's running maximum jumped by tens of nats
 *                            while the other's did not
 *   flags_out   device uint8[n_rows], owned by the caller
 * Asynchronous on `stream`, ordered after earlier kld_eval_rows calls on any
 * stream. Returns KLD_ERR_INVALID_ARG for a NULL flags_out (with n_rows > 0)
 * or negative counts, KLD_ERR_RANGE when row_offset + n_rows > max_rows,
 * KLD_ERR_HIP if the copy fails.
 */
enum {
    KLD_ROW_FLAG_AMPLIFIED = 1,
    KLD_ROW_FLAG_QUANT_MASS = 2,
    KLD_ROW_FLAG_CARRIED = 4
};
kld_status kld_eval_copy_row_flags(kld_eval* h, int64_t row_offset, int64_t n_rows, uint8_t* flags_out,
                                   void* stream);

/*
 * Gradient of the per-token KL(P_base || Q_quant) with respect to the
 * quantized logits: grad[r][i] = scale * (q_i - p_i), where p and q are the
 * softmaxes of base row r and quant row r (the derivative of the log-sum-exp
 * is the softmax). This is the first step of the backward pass of the loss the
 * GSQ-RCO model card's end-to-end tuning minimises, KL(BF16 || quantized) of
 * the next-token distributions ("How it was made" step 7); `scale` is the
 * row's weight in that loss (1/N for the mean over N rows).
 *   base, quant  the same rows that kld_eval_rows evaluated into handle rows
 *                [row_offset, row_offset + n_rows): the float64
 *                log-normalisers saved there are reused, so this call reads
 *                the rows once more and needs no reduction
 *   grad_out     device [n_rows, vocab] row-major array of grad_dtype
 *                (KLD_DTYPE_F32, or KLD_DTYPE_BF16 rounded to nearest even),
 *                owned by the caller
 * Asynchronous on `stream`, ordered after earlier kld_eval_rows calls on any
 * stream. Rows overwritten by a later kld_eval_rows before this call's work
 * runs give undefined gradients. Returns KLD_ERR_INVALID_ARG for NULL
 * pointers, a bad grad_dtype or a non-finite scale, KLD_ERR_RANGE when
 * row_offset + n_rows > max_rows, KLD_ERR_HIP if the launch fails.
 */
kld_status kld_eval_grad(kld_eval* h, const void* base, const void* quant, int64_t n_rows,
                         int64_t row_offset, double scale, void* grad_out, int32_t grad_dtype,
                         void* stream);

/*
 * Base rows stored as their top-K tokens plus the rest of the mass -- the form
 * the GSQ-RCO model card tunes against ("How it was made" step 7: the BF16
 * model's top-128 distributions and the rest of the mass).
 *
 * kld_eval_topk_compress: for each of n_rows base rows ([n_rows, vocab] device
 * array of the handle's base dtype) store
 *   idx_out   int32[n_rows][k]  the k largest logits' indices, most probable
 *                               first, equal logits by lowest index (+0 and -0
 *                               are equal), so idx_out[r][0] is the argmax
 *   logp_out  float32[n_rows][k] their log-probabilities z - lse
 *   rest_out  float32[n_rows]   the probability of every other token, summed
 *                               over those tokens (0 when k == vocab)
 * k in [1, min(vocab, 1024)]. Device arrays, owned by the caller; handle rows
 * are not touched. Asynchronous on `stream`. Deterministic.
 *
 * kld_eval_rows_topk: like kld_eval_rows, with the base given in that stored
 * form (the same k) and the quantized rows in full ([n_rows, vocab] of the
 * handle's quant dtype). Per row it computes the KL divergence of both
 * distributions coarsened to the k stored tokens plus one outcome "any other
 * token":
 *   KL_k = sum_j p_j (log p_j - log q_j) + R (log R - log Q_rest)
 * (p_j = exp(logp[j]), R = rest; q_j, Q_rest from the quantized row; a term
 * with R == 0 is 0) -- the full KL when k == vocab, never more than it
 * otherwise -- and the top-1 match of the quantized argmax (lowest index)
 * with idx[0]. Results go to handle rows [row_offset, row_offset + n_rows)
 * exactly as kld_eval_rows writes them (kld, match, argmax_base = idx[0],
 * argmax_quant, log-normaliser of the quant row; the base log-normaliser is
 * NaN and no token is scored), so kld_eval_reduce and the segmented reduction
 * summarize them. Stored indices must be distinct and in [0, vocab): a row
 * that breaks this gets a NaN divergence and match 0. Needs vocab / 8 bytes of
 * on-chip memory per workgroup: KLD_ERR_INVALID_ARG when the device has too
 * little (vocab beyond about one million on gfx950).
 * Both return KLD_ERR_INVALID_ARG for NULL pointers, negative counts or a bad
 * k, KLD_ERR_RANGE when row_offset + n_rows > max_rows, KLD_ERR_HIP if a
 * launch fails.
 */
kld_status kld_eval_topk_compress(kld_eval* h, const void* base, int64_t n_rows, int32_t k,
                                  int32_t* idx_out, float* logp_out, float* rest_out, void* stream);

kld_status kld_eval_rows_topk(kld_eval* h, const int32_t* topk_idx, const float* topk_logp,
                              const float* topk_rest, int32_t k, const void* quant,
                              int64_t n_rows, int64_t row_offset,
                              float* kld_out, uint8_t* match_out,
                              int32_t* argmax_base_out, int32_t* argmax_quant_out,
                              void* stream);

/*
 * Gradient of the coarsened divergence KL_k of kld_eval_rows_topk with respect
 * to the quantized logits, the stored form held fixed -- the first step of the
 * backward pass of the GSQ-RCO model card's tuning phase against the top-128
 * distributions and the rest of the mass ("How it was made" step 7). With q the
 * quantized softmax, S the stored tokens, P = sum_j p_j, R = rest and Q_rest
 * the quantized mass outside S:
 *   grad[r][i] = scale * (q_i (P + R) - p_i)                 for i in S
 *   grad[r][i] = scale * q_i (P + R - R / Q_rest)            otherwise
 * (q - p when k == vocab). `scale` is the row's weight in the loss.
 *   topk_idx, topk_logp, k, quant
 *                the stored indices and log-probabilities and the quantized
 *                rows that kld_eval_rows_topk evaluated into handle rows
 *                [row_offset, row_offset + n_rows): the quant log-normaliser
 *                and the factors P + R and P + R - R / Q_rest that call saved
 *                there are reused (R enters only through them), so this call
 *                reads each quant row once more; rows last written by
 *                kld_eval_rows hold no such factors and give undefined
 *                gradients
 *   grad_out     device [n_rows, vocab] row-major array of grad_dtype
 *                (KLD_DTYPE_F32, or KLD_DTYPE_BF16 rounded to nearest even),
 *                owned by the caller; every entry is written
 * A row whose stored indices are not distinct and in [0, vocab) is written as
 * NaN. Asynchronous on `stream`, ordered after earlier calls on any stream.
 * Returns KLD_ERR_INVALID_ARG for NULL pointers, a bad k or grad_dtype or a
 * non-finite scale, KLD_ERR_RANGE when row_offset + n_rows > max_rows,
 * KLD_ERR_HIP if the launch fails.
 */
kld_status kld_eval_grad_topk(kld_eval* h, const int32_t* topk_idx, const float* topk_logp, int32_t k,
                              const void* quant, int64_t n_rows, int64_t row_offset, double scale,
                              void* grad_out, int32_t grad_dtype, void* stream);

/*
 * Measurement aid, not a step of the method: the attainable HBM read rate for
 * the row kernels' access pattern, to set their timing against. Reads n_rows
 * rows of row_bytes bytes from `a` (and, when `b` is not NULL, the same rows
 * of `b`) once, one workgroup of waves_per_row waves (1 or 4) per row,
 * 16-byte non-temporal loads from 1 KiB tiles, four tiles per row in flight
 * per wave -- the row kernel's load shapes with no arithmetic -- and writes
 * sink[r] = the XOR of every 32-bit word of row r of a (and b), so that the
 * reads are not removed and can be checked. Device pointers on the current
 * device; a, b 16-byte aligned, row_bytes a positive multiple of 16; sink is
 * uint32[n_rows], owned by the caller. Asynchronous on `stream`; no handle is
 * involved. start_event / stop_event (hipEvent_t as void*, each may be NULL,
 * created by the caller with timing): recorded by the probe's first launch
 * when it begins and by its last when it ends, as kld_eval_rows_timed does,
 * so the probe and the row pass are timed the same way. Returns
 * KLD_ERR_INVALID_ARG for NULL a or sink, negative n_rows, a bad row_bytes or
 * waves_per_row or misaligned pointers, KLD_ERR_HIP if the launch fails.
 */
kld_status kld_eval_read_probe(const void* a, const void* b, int64_t n_rows, int64_t row_bytes,
                               int32_t waves_per_row, uint32_t* sink, void* stream,
                               void* start_event, void* stop_event);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The same
 * comparison as kld_eval_rows over rows [0, n_rows) followed by
 * kld_eval_reduce, with no handle: it calls no allocator, enqueues everything
 * on `stream` and never blocks.
 *   base, quant   device [n_rows, vocab] arrays of base_dtype / quant_dtype
 *   kld_out       float32[n_rows], required (the reduction reads it)
 *   match_out     uint8[n_rows], required (the reduction reads it)
 *   argmax_base_out, argmax_quant_out   int32[n_rows], optional (NULL skips)
 *   summary_out   device memory for one kld_eval_summary, written by the
 *                 last kernel of the call; read it after the stream reaches
 *                 that point
 * The results are bit-identical to kld_eval_rows + kld_eval_reduce on a
 * handle created with max_rows = n_rows. The reduction's partials live in a
 * fixed workspace inside the library, one per GPU, sized for at most
 * 4,194,304 rows (320 KiB); calls on one GPU share it, so calls that overlap
 * on one GPU (two streams, or two threads) race and must be serialised by the
 * caller. Needs a gfx950 as the current device.
 * Returns KLD_ERR_INVALID_ARG for NULL required pointers, a bad vocab or
 * dtype, or negative n_rows; KLD_ERR_EMPTY for n_rows == 0; KLD_ERR_RANGE for
 * n_rows > 4194304; KLD_ERR_UNSUPPORTED_ARCH / KLD_ERR_NO_DEVICE for the
 * device; KLD_ERR_HIP if a launch fails.
 */
kld_status kld_eval_compare_noalloc(const void* base, const void* quant, int64_t vocab, int64_t n_rows,
                                    int32_t base_dtype, int32_t quant_dtype,
                                    float* kld_out, uint8_t* match_out,
                                    int32_t* argmax_base_out, int32_t* argmax_quant_out,
                                    kld_eval_summary* summary_out, void* stream);

/* Synchronize the handle's work and free it. NULL is a no-op returning KLD_OK. */
kld_status kld_eval_destroy(kld_eval* h);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* kld_eval_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KLD_EVAL_H */
