/*
 * attn.h -- C ABI of libattn.so: exact attention with an online softmax on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones described on the pofe.ai page "FlashAttention
 * for inference: tiled prefill and split-KV decoding":
 *   - attn_prefill: tiled causal (or full) prefill; query tiles walk key/value
 *     tiles, scores stay on chip, each row keeps a running max and sum, and
 *     the row log-sum-exp is written out (sections "The online softmax, with
 *     every symbol defined" and "Prefill: tiles, loop order and the tensor
 *     cores");
 *   - attn_prefill_varlen: the same over a packed batch of sequences of
 *     different lengths (cumulative offsets, no padding);
 *   - attn_decode: one query token per sequence against a paged (or
 *     contiguous) KV cache, the keys split into chunks processed by separate
 *     workgroups, each chunk's (output, log-sum-exp) merged by a separate
 *     reduction (section "Decode: a different bottleneck"; layouts from
 *     section "Minimal implementation");
 *   - attn_decode_append: the same decode step with the new token's key and
 *     value written into the cache in place first (section "Minimal
 *     implementation");
 *   - attn_prefill_ext / attn_decode_ext: the same operations with a sliding
 *     window and logit soft-capping, two of the attention variants the
 *     page's section "Interaction with post-trained models" names as ones a
 *     kernel has to support;
 *   - attn_prefill_fp8: the prefill on 8-bit (E4M3) inputs with descale
 *     factors, the FP8 direction the page names for FlashAttention-3 (section
 *     "The bottleneck it attacks");
 *   - attn_prefill_fp8_varlen: the FP8 prefill over a packed batch;
 *   - attn_decode_fp8: the decode over an FP8 (E4M3) KV cache;
 *   - attn_decode_fp8_append: the same with the new token's codes appended in place;
 *   - attn_decode_noalloc: attn_decode with its partials in a static device
 *     array, for callers that cannot allocate;
 *   - attn_lse_combine: that reduction on its own -- the combine rule for
 *     independent partials, a softmax over the partials' log-sum-exps
 *     (section "The online softmax, with every symbol defined" and the
 *     `merge` helper of section "Minimal implementation").
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer owned by the caller; the
 *     library allocates nothing, keeps no state between calls and is safe to
 *     call from several host threads.  (One exception: attn_decode_noalloc keeps
 *     its partials in a static per-GPU device array, so its calls that overlap
 *     on one GPU race; see there.)  Tensors are dense, row-major, with the
 *     layouts stated per call, and must be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream).  Nothing synchronises with the host.
 *   - Return value: ATTN_OK (0) or a negative status.  Argument errors are
 *     detected on the host before any HIP call, so they are reported even on a
 *     machine without a GPU.  A failed launch is reported as ATTN_ERR_HIP.
 *     There is no silent fallback to another algorithm or precision: a shape,
 *     dtype or head size the kernels do not implement is ATTN_ERR_UNSUPPORTED.
 *   - Values the host cannot see (seq_lens and block_table contents) are the
 *     caller's responsibility: each seq_lens[b] must lie in
 *     [0, max_blocks_per_seq * page_size] (the kernels clamp a value outside
 *     that range into it rather than read past the cache) and each
 *     block-table entry a sequence reaches must name a page of the cache.
 *   - Scores are s = scale * <q, k>; LSE outputs are natural logarithms over
 *     scaled scores, lse = m + ln(l).  A row with no visible key gets O = 0 and
 *     LSE = -inf.
 *   - Grouped-query attention: query head h reads KV head h / (n_q_heads /
 *     n_kv_heads) (consecutive query heads share a KV head).
 *   - Head sizes 64, 128 and 256 (256 being the largest the page's section
 *     "Interaction with post-trained models" names) on every entry point except
 *     the E4M3-cache decodes (attn_decode_fp8, attn_decode_fp8_append,
 *     attn_decode_fp8_ext: 64 and 128).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define ATTN_OK               0
#define ATTN_ERR_NULL        -1  /* a required pointer is NULL                          */
#define ATTN_ERR_SHAPE       -2  /* a size is <= 0 (or negative where 0 is allowed)     */
#define ATTN_ERR_GQA         -3  /* n_q_heads is not a multiple of n_kv_heads            */
#define ATTN_ERR_UNSUPPORTED -4  /* head_dim, dtype, group size or chunk not implemented */
#define ATTN_ERR_WORKSPACE   -5  /* workspace NULL or smaller than required             */
#define ATTN_ERR_ALIGN       -6  /* a tensor pointer is not 16-byte aligned             */
#define ATTN_ERR_HIP         -7  /* the HIP runtime reported an error at launch          */
#define ATTN_ERR_SCRATCH     -8  /* attn_decode_noalloc: partials exceed its static scratch */

/* ---- element types ----------------------------------------------------- */
#define ATTN_F32  0  /* IEEE binary32                                   */
#define ATTN_BF16 1  /* bfloat16 (upper half of binary32), stored 2 B   */

/*
 * attn_prefill -- exact attention for a whole prompt, O = softmax(scale*QK^T) V.
 *
 *   q    [batch, n_q_heads,  seqlen, head_dim]  element type `dtype`
 *   k, v [batch, n_kv_heads, seqlen, head_dim]  element type `dtype`
 *   o    [batch, n_q_heads,  seqlen, head_dim]  element type `dtype` (written)
 *   lse  [batch, n_q_heads,  seqlen] float32, row log-sum-exp (written; required)
 *   causal != 0: row i attends keys 0..i; causal == 0: all keys.
 *   head_dim in {64, 128, 256}; dtype ATTN_BF16 (matrix cores, bf16 products with
 *   float32 accumulation; P is rounded to bf16 before the P*V product; O is
 *   rounded to nearest even) or ATTN_F32 (float32 arithmetic throughout).
 *   batch, seqlen >= 0 (an empty call does nothing); heads >= 1;
 *   (seqlen + 255) * head_dim * 2 >= 2^32 is ATTN_ERR_UNSUPPORTED.
 */
int attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse,
                 int batch, int seqlen, int n_q_heads, int n_kv_heads, int head_dim,
                 int dtype, int causal, float scale, void *stream);

/*
 * attn_prefill_varlen -- attn_prefill over a packed batch of sequences of
 * different lengths, without padding: engines batch prompts this way through
 * a variable-length interface (pofe.ai page, section "Interaction with
 * post-trained models").  Sequence b owns tokens cu_seqlens[b] ..
 * cu_seqlens[b+1]-1; each sequence attends only to itself (causal within it).
 *
 *   q, o  [total_tokens, n_q_heads,  head_dim]  element type `dtype`
 *   k, v  [total_tokens, n_kv_heads, head_dim]  element type `dtype`
 *   lse   [n_q_heads, total_tokens] float32 (written; required)
 *   cu_seqlens [batch + 1] int32 on the device: cu_seqlens[0] = 0, nondecreasing,
 *         cu_seqlens[batch] = total_tokens (4-byte aligned)
 *   max_seqlen >= every cu_seqlens[b+1] - cu_seqlens[b]; it sizes the launch.
 *   The device-side offsets are the caller's responsibility; an offset outside
 *   [0, total_tokens] or a length above max_seqlen is clamped (nothing outside the
 *   tensors is touched, but those rows are not computed as intended).
 *   dtype, head_dim, causal and scale as attn_prefill; same element arithmetic.
 *   Larger than (max_seqlen + 255) * n_q_heads * head_dim * element size >= 2^32 is
 *   ATTN_ERR_UNSUPPORTED.  batch, max_seqlen or total_tokens of 0 does nothing.
 */
int attn_prefill_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *cu_seqlens, int batch, int max_seqlen, int total_tokens,
                        int n_q_heads, int n_kv_heads, int head_dim, int dtype, int causal, float scale,
                        void *stream);

/*
 * attn_prefill_ext -- attn_prefill (cu_seqlens_or_null == NULL; seqlen is N and
 * total_tokens is ignored) or attn_prefill_varlen (cu_seqlens_or_null != NULL;
 * seqlen is max_seqlen), with two options:
 *
 *   window_left  -1: no window.  >= 0: the query at position i of its sequence
 *                also needs key position j >= i - window_left (a sliding window
 *                of window_left + 1 keys when causal; without causal, keys
 *                i - window_left .. end).  Below -1 is ATTN_ERR_SHAPE.
 *   softcap      0: none.  > 0 (finite): each score s = scale * <q, k> becomes
 *                softcap * tanh(s / softcap) before masking and the softmax;
 *                negative or non-finite is ATTN_ERR_SHAPE.  dtype ATTN_BF16
 *                forms tanh(y) as 1 - 2 / (e^{2y} + 1) with the hardware
 *                exponential and reciprocal (about 1e-7 * softcap absolute error
 *                in a score); ATTN_F32 calls the device library's tanhf.
 *   Every row still sees at least its own key (causal) or the last key, so no
 *   row is empty.  With window_left = -1 and softcap = 0 the results are those
 *   of attn_prefill / attn_prefill_varlen (the same kernels run).  Layouts,
 *   element arithmetic, limits and errors as those two calls.
 */
int attn_prefill_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                     const int32_t *cu_seqlens_or_null, int batch, int seqlen, int total_tokens,
                     int n_q_heads, int n_kv_heads, int head_dim, int dtype, int causal, float scale,
                     int window_left, float softcap, void *stream);

/*
 * attn_prefill_fp8 -- attn_prefill on FP8 inputs: O = softmax(s) V with scores
 * s = scale * descale_q * descale_k * <q8, k8> and values descale_v * v8.
 *
 *   q    [batch, n_q_heads,  seqlen, head_dim]  E4M3 codes (OCP 8-bit float,
 *        finite-only variant: bias 7, max 448), one byte each
 *   k, v [batch, n_kv_heads, seqlen, head_dim]  E4M3 codes
 *   o    [batch, n_q_heads,  seqlen, head_dim]  bfloat16 (written)
 *   lse  [batch, n_q_heads,  seqlen] float32, natural log over the scaled scores
 *   descale_q/k/v_or_null [batch, n_kv_heads] float32 on the device, 4-byte
 *        aligned, one factor per (sequence, KV head) shared by the group's query
 *        heads; NULL means 1.
 *   head_dim in {64, 128, 256}; causal and scale as attn_prefill.  Arithmetic: both
 *   products on the FP8 matrix cores with float32 accumulation; the
 *   probabilities are rounded to E4M3 (nearest even, each <= 256) before the
 *   P*V product, so O carries up to 2^-4 relative error per term (2^-10
 *   absolute below E4M3's normal range); the row sums and the LSE use the
 *   unrounded float32 values.  NaN codes (0x7f, 0xff) in the inputs are the
 *   caller's error.  (seqlen + 127) * head_dim >= 2^32 is ATTN_ERR_UNSUPPORTED.
 */
int attn_prefill_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                     const float *descale_q_or_null, const float *descale_k_or_null,
                     const float *descale_v_or_null, int batch, int seqlen, int n_q_heads, int n_kv_heads,
                     int head_dim, int causal, float scale, void *stream);

/*
 * attn_prefill_fp8_varlen -- attn_prefill_fp8 over a packed batch of sequences
 * (the layout of attn_prefill_varlen).  The pofe.ai page's section
 * "Interaction with post-trained models" discusses both FP8 attention and the
 * variable-length interface engines use to batch prompts without padding.
 * Sequence b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 and attends only
 * to itself.
 *
 *   q     [total_tokens, n_q_heads,  head_dim]  E4M3 codes
 *   k, v  [total_tokens, n_kv_heads, head_dim]  E4M3 codes
 *   o     [total_tokens, n_q_heads,  head_dim]  bfloat16 (written)
 *   lse   [n_q_heads, total_tokens] float32 (written)
 *   descale_q/k/v_or_null [batch, n_kv_heads] float32, one factor per (sequence,
 *         KV head); NULL means 1.
 *   cu_seqlens, max_seqlen: as attn_prefill_varlen (offsets outside
 *         [0, total_tokens] or lengths above max_seqlen are clamped).
 *   head_dim in {64, 128, 256}; arithmetic as attn_prefill_fp8.
 *   (max_seqlen + 127) * n_q_heads * head_dim >= 2^32 is ATTN_ERR_UNSUPPORTED;
 *   batch, max_seqlen or total_tokens of 0 does nothing.
 */
int attn_prefill_fp8_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                            const float *descale_q_or_null, const float *descale_k_or_null,
                            const float *descale_v_or_null, const int32_t *cu_seqlens, int batch,
                            int max_seqlen, int total_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                            int causal, float scale, void *stream);

/*
 * attn_prefill_fp8_ext -- attn_prefill_fp8 (cu_seqlens_or_null == NULL; seqlen is
 * N, total_tokens ignored) or attn_prefill_fp8_varlen (cu_seqlens_or_null !=
 * NULL; seqlen is max_seqlen) with the sliding window and the logit soft-cap of
 * attn_prefill_ext, the two variants the pofe.ai page's section "Interaction
 * with post-trained models" lists, on 8-bit inputs as that section's FP8
 * paragraph describes.
 *
 *   window_left  -1: no window; >= 0: the query at position i also needs key
 *                position j >= i - window_left; below -1 is ATTN_ERR_SHAPE.
 *   softcap      0: none; > 0 (finite): each scaled score s = scale * dq * dk *
 *                <q8, k8> becomes softcap * tanh(s / softcap) before masking and
 *                the softmax (tanh(y) formed as 1 - 2 / (e^{2y} + 1) with the
 *                hardware exponential and reciprocal); negative or non-finite is
 *                ATTN_ERR_SHAPE.
 *   With window_left = -1 and softcap = 0 the plain FP8 kernels run (the results
 *   of attn_prefill_fp8 / attn_prefill_fp8_varlen, bit for bit).  Layouts,
 *   descales, arithmetic, limits and errors as those two calls.
 */
int attn_prefill_fp8_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                         const float *descale_q_or_null, const float *descale_k_or_null,
                         const float *descale_v_or_null, const int32_t *cu_seqlens_or_null, int batch, int seqlen,
                         int total_tokens, int n_q_heads, int n_kv_heads, int head_dim, int causal, float scale,
                         int window_left, float softcap, void *stream);

/*
 * attn_decode -- one new query token per sequence against a KV cache, by
 * split-KV: the first seq_lens[b] tokens of sequence b are cut into chunks of
 * `chunk_tokens`; one workgroup per (sequence, KV head, chunk) computes the
 * chunk's normalised output and log-sum-exp for all query heads of that KV
 * head; a second kernel merges the chunks with the combine rule.  With
 * chunk_tokens == 0 and batch >= 2 the split is balanced instead: each KV head's
 * tokens of all sequences, in sequence order and in units of one workgroup pass
 * (256 tokens; 128 at head_dim 256), are cut into 256 / n_kv_heads equal
 * contiguous shares (256 workgroups in all, one per compute unit), and a
 * workgroup writes one partial for every sequence its share touches, so a batch
 * of mixed lengths keeps every workgroup busy to the end.  The pieces are found
 * on the device from seq_lens; the combine rule is the same, only the grouping of
 * the keys (and so the float32 rounding) differs between the two splits.
 *
 *   q        [batch, n_q_heads, head_dim]                      element `dtype`
 *   k_cache, v_cache:
 *     paged      (block_table != NULL): [num_pages, page_size, n_kv_heads, head_dim]
 *     contiguous (block_table == NULL): [batch, max_blocks_per_seq*page_size,
 *                                        n_kv_heads, head_dim]
 *   block_table [batch, max_blocks_per_seq] int32: token t of sequence b is
 *               slot t % page_size of page block_table[b][t / page_size]
 *   seq_lens    [batch] int32: number of cached tokens the query attends
 *               (already including the new token's own key/value)
 *   o           [batch, n_q_heads, head_dim]  element `dtype` (written)
 *   lse_or_null [batch, n_q_heads] float32 (written when not NULL)
 *   chunk_tokens: 0 = balanced split for batch >= 2, else a chunk chosen from
 *               batch, heads and capacity (attn_decode_chunk_tokens);
 *               otherwise a positive multiple of 16 (one workgroup per chunk).
 *   workspace / workspace_bytes: device scratch of at least
 *               attn_decode_workspace_bytes(...) bytes for the partials;
 *               contents on entry are ignored.
 *   Size limits (else ATTN_ERR_UNSUPPORTED): batch <= 65535, batch*n_q_heads < 2^24,
 *   chunks per sequence < 2^22 and chunks per sequence * n_kv_heads < 2^23.
 *   head_dim in {64, 128, 256}; n_q_heads / n_kv_heads <= 16; dtype ATTN_BF16 only
 *   (bf16 products on matrix cores with float32 accumulation, P rounded to bf16
 *   before the P*V product, partials and the combine in float32, O rounded to
 *   nearest even).  A paged cache needs page_size a multiple of 16 (no 16-token
 *   block straddles two pages); for a contiguous cache page_size only sets the
 *   capacity max_blocks_per_seq * page_size.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_table, const int32_t *seq_lens, void *o,
                float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                int page_size, int max_blocks_per_seq, int dtype, float scale,
                int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_noalloc -- attn_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The per-chunk partials go to a static device
 * array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU,
 * which each GPU the library runs on holds until the process ends; its address is
 * looked up once per device (with that device current) on the first call there.
 * The call allocates nothing: no hipMalloc, hipFree or allocating library routine.
 *
 *   Arguments, layouts, arithmetic, limits and results are those of attn_decode
 *   (the same kernels run; the outputs are bit for bit those of attn_decode),
 *   except that a balanced split (chunk_tokens == 0, batch >= 2) whose partials
 *   do not fit the array runs as the per-chunk split of the automatic chunk size
 *   (attn_decode_chunk_tokens) instead, whose rounding differs.  A call whose
 *   partials, per-chunk split included, exceed ATTN_DECODE_NOALLOC_SCRATCH_BYTES
 *   is ATTN_ERR_SCRATCH (checked on the host, before any HIP call).  The scratch keeps the last call's partials; nothing in
 *   it needs to start at zero (every partial the combine weighs is written first).
 *   Calls on one GPU share that GPU's array: calls that may overlap in time (on
 *   different streams, or from several host threads without ordering) race on it
 *   and must be serialised by the caller, e.g. by issuing them on one stream.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *block_table, const int32_t *seq_lens, void *o,
                        float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                        int page_size, int max_blocks_per_seq, int dtype, float scale,
                        int chunk_tokens, void *stream);

/*
 * attn_decode_append -- attn_decode with the new token's key and value appended
 * to the cache in place first, as the decode step of the pofe.ai page's section
 * "Minimal implementation" does: cache_seqlens counts the tokens already cached
 * (before the new one); the new rows are written at token cache_seqlens[b] of
 * sequence b (slot cache_seqlens[b] % page_size of page
 * block_table[b][cache_seqlens[b] / page_size], or row cache_seqlens[b] of a
 * contiguous cache), and the query attends cache_seqlens[b] + 1 tokens.
 *
 *   k_new, v_new [batch, n_kv_heads, head_dim]  element `dtype` (read)
 *   k_cache, v_cache: as attn_decode, written at the new token's slot only
 *   cache_seqlens [batch] int32, read only: the caller advances it afterwards
 *   All other arguments, the workspace and the limits are those of attn_decode.
 *   Each cache_seqlens[b] must be below max_blocks_per_seq * page_size and the
 *   block-table entry of the new token must name a page of the cache; a value
 *   outside [0, capacity - 1] is clamped into it (a full cache's new row lands
 *   in its last slot).  k_new and v_new are required (ATTN_ERR_NULL).
 */
int attn_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *block_table, const int32_t *cache_seqlens, void *o,
                       float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                       int page_size, int max_blocks_per_seq, int dtype, float scale, int chunk_tokens,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_ext -- attn_decode (k_new_or_null and v_new_or_null both NULL) or
 * attn_decode_append (both set; one of them NULL is ATTN_ERR_NULL), with the
 * options of attn_prefill_ext: the query is token L - 1 of its sequence, where L
 * is the number of tokens it attends (seq_lens[b], or cache_seqlens[b] + 1 with
 * the append), so window_left >= 0 limits it to tokens L - 1 - window_left ..
 * L - 1 (chunks wholly before that are not read); softcap > 0 caps every score
 * as in attn_prefill_ext (hardware exponential and reciprocal).  Arguments,
 * workspace, layouts and limits as attn_decode / attn_decode_append.
 */
int attn_decode_ext(const void *q, const void *k_new_or_null, const void *v_new_or_null, void *k_cache,
                    void *v_cache, const int32_t *block_table, const int32_t *seq_lens, void *o,
                    float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                    int max_blocks_per_seq, int dtype, float scale, int window_left, float softcap,
                    int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_fp8 -- attn_decode over an FP8 KV cache: k_cache and v_cache hold
 * E4M3 codes (one byte per element, same layouts as attn_decode), the values being
 * descale_k * k8 and descale_v * v8 with one factor per (sequence, KV head)
 * ([batch, n_kv_heads] float32 on the device, 4-byte aligned; NULL means 1).  The
 * decode split of the pofe.ai page's section "Decode: a different bottleneck" reads
 * half the bytes per token of a bf16 cache.  q and o are bfloat16 as in
 * attn_decode.  The codes convert to bf16 exactly; the products and the combine
 * are those of attn_decode, with descale_k folded into the score scale and
 * descale_v into the output.  head_dim 64 or 128 (else ATTN_ERR_UNSUPPORTED); no
 * append, window or soft-cap.  Workspace, chunking and limits as attn_decode.
 */
int attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache, const float *descale_k_or_null,
                    const float *descale_v_or_null, const int32_t *block_table, const int32_t *seq_lens, void *o,
                    float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                    int max_blocks_per_seq, float scale, int chunk_tokens, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * attn_decode_fp8_append -- attn_decode_fp8 with the new token's key and value
 * written into the E4M3 cache in place first: the decode step of the pofe.ai
 * page's section "Minimal implementation" (the cache takes the new rows, then the
 * query attends them) on the 8-bit cache whose half-size rows section "Decode: a
 * different bottleneck" says decode is bound by.
 *
 *   k_new, v_new [batch, n_kv_heads, head_dim]  E4M3 codes, one byte each, already
 *                quantised with the cache's descales (value = descale * code);
 *                written unchanged at token cache_seqlens[b] of sequence b, exactly as
 *                attn_decode_append places its rows (slot t % page_size of page
 *                block_table[b][t / page_size], or row t of a contiguous cache; t
 *                clamped into [0, capacity - 1])
 *   cache_seqlens [batch] int32, read only: tokens already cached; the query
 *                attends cache_seqlens[b] + 1 tokens and the caller advances it
 *   Every other argument, the descales, head sizes (64, 128), workspace, limits and
 *   errors are those of attn_decode_fp8; k_new and v_new are required (ATTN_ERR_NULL)
 *   and 16-byte aligned (ATTN_ERR_ALIGN).  No window or soft-cap.
 */
int attn_decode_fp8_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const float *descale_k_or_null, const float *descale_v_or_null, const int32_t *block_table,
                           const int32_t *cache_seqlens, void *o, float *lse_or_null, int batch, int n_q_heads,
                           int n_kv_heads, int head_dim, int page_size, int max_blocks_per_seq, float scale,
                           int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_fp8_ext -- attn_decode_fp8 with the sliding window and the logit
 * soft-cap of attn_decode_ext (window_left: the query, token L-1, also needs
 * token j >= L-1-window_left, -1 = none; softcap > 0 caps each scaled score
 * s = scale * descale_k * <q, k8> at softcap * tanh(s / softcap), 0 = none; the
 * variants of the pofe.ai page's section "Interaction with post-trained
 * models").  With window_left = -1 and softcap = 0 the attn_decode_fp8 kernel
 * runs (bit for bit).  Every other argument, the workspace, the limits and the
 * errors are those of attn_decode_fp8; window_left below -1 or a negative or
 * non-finite softcap is ATTN_ERR_SHAPE.
 */
int attn_decode_fp8_ext(const void *q, const void *k_cache, const void *v_cache, const float *descale_k_or_null,
                        const float *descale_v_or_null, const int32_t *block_table, const int32_t *seq_lens, void *o,
                        float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                        int max_blocks_per_seq, float scale, int window_left, float softcap, int chunk_tokens,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_chunk_tokens -- the chunk size of the per-chunk split for these
 * arguments (resolves chunk_tokens == 0; attn_decode uses it for batch 1 and with
 * a window or soft-cap, the balanced split otherwise), or a negative status.
 */
int attn_decode_chunk_tokens(int batch, int n_kv_heads, int page_size, int max_blocks_per_seq,
                             int chunk_tokens);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace the split-KV decode
 * needs for its per-chunk partials: each chunk of a sequence's keys yields a
 * normalised partial output and its log-sum-exp, which the separate combine then
 * merges (pofe.ai page, section "Decode: a different bottleneck").  The size is
 *   batch * n_q_heads * splits * (head_dim + 1) * 4
 * (partials are float32), where splits = ceil(max_blocks_per_seq * page_size /
 * chunk) with chunk the chunk size attn_decode_chunk_tokens resolves; with
 * chunk_tokens == 0 and batch >= 2, splits is the larger of that and the balanced
 * split's bound min(256 / n_kv_heads, ceil(capacity / unit)), unit 256 tokens
 * (128 at head_dim 256).  0 if the arguments are invalid.
 * The arguments are those of attn_decode that fix the chunk count: the capacity
 * max_blocks_per_seq * page_size bounds every sequence's length, and n_kv_heads
 * and page_size enter the automatic chunk choice (chunk_tokens == 0).  Pure host
 * function: no HIP call, callable without a GPU.
 */
size_t attn_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                   int page_size, int max_blocks_per_seq, int chunk_tokens);

/*
 * attn_lse_combine -- merge independent partial results of the same rows:
 * Lambda = ln sum_k exp(lambda_k), o = sum_k exp(lambda_k - Lambda) o_k.
 *
 *   o_parts   [rows, max_splits, head_dim] float32 (normalised partial outputs)
 *   lse_parts [rows, max_splits] float32 (their log-sum-exps; -inf = empty)
 *   n_splits_or_null [rows] int32: use the first n_splits[r] partials of row r
 *               (0 <= n <= max_splits); NULL = all max_splits
 *   o         [rows, head_dim] element type `o_dtype` (ATTN_F32 or ATTN_BF16)
 *   lse_or_null [rows] float32 (written when not NULL)
 *   A row whose partials are all empty gets o = 0, Lambda = -inf.
 *   head_dim in {64, 128, 256}; rows >= 0; 1 <= max_splits < 2^22 and rows < 2^24
 *   (larger is ATTN_ERR_UNSUPPORTED).
 */
int attn_lse_combine(const float *o_parts, const float *lse_parts,
                     const int32_t *n_splits_or_null, int rows, int max_splits, int head_dim,
                     void *o, int o_dtype, float *lse_or_null, void *stream);

/*
 * attn_decode_check_tables -- count, on the device, the entries of a decode's
 * block table and lengths that would send attn_decode (or attn_decode_append)
 * outside the cache.  The page's section "Minimal implementation" defines the
 * paged cache (num_blocks, block_size, kv_heads, head_dim), the block table
 * (batch, max_blocks) int32 and the per-sequence lengths; the decode kernels read
 * these device arrays without checking them, since the host cannot see them.
 * Callers that build tables from untrusted or changing state can run this first
 * (a debug mode), synchronise, and read the count.
 *
 *   block_table_or_null [batch, max_blocks_per_seq] int32, or NULL for a
 *               contiguous cache (only the lengths are checked)
 *   seq_lens    [batch] int32: the lengths attn_decode would be given
 *   num_blocks  pages in the cache pool (entries must lie in [0, num_blocks))
 *   appended    0: lengths count the attended tokens (attn_decode); 1: lengths
 *               count the cached tokens before an in-place append
 *               (attn_decode_append), so one more token must fit
 *   bad_out     one int32 on the device, overwritten with the count: each
 *               sequence with length < 0 or length + appended > max_blocks_per_seq
 *               * page_size counts once, and each table slot j with j * page_size
 *               < min(length + appended, capacity) holding an entry outside [0,
 *               num_blocks) counts once (slots past a sequence's length are never
 *               read and are not checked); saturates at INT32_MAX.
 *   All pointers are device pointers, 4-byte aligned (else ATTN_ERR_ALIGN);
 *   bad_out may not be NULL, nor seq_lens unless batch is 0 (which writes 0).  Asynchronous on
 *   `stream`; one workgroup reads each length and table entry once; no memory
 *   other than *bad_out is written.
 */
int attn_decode_check_tables(const int32_t *block_table_or_null, const int32_t *seq_lens, int batch,
                             int page_size, int max_blocks_per_seq, int num_blocks, int appended,
                             int32_t *bad_out, void *stream);

/* attn_status_string -- static, human-readable text for a status code. */
const char *attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
