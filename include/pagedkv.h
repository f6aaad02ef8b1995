/*
 * pagedkv.h -- C ABI of libpagedkv.so: decode-step attention over a paged
 * KV cache on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [A] "KV-Cache Engineering: Paged Attention, Prefix Cache,
 *        Disaggregation (2026)".
 *   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
 *        Attention Variants, and the Bandwidth Wall".
 *   [C] "KV-Cache Engineering: The Memory Wall of LLM Serving".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Every tensor pointer is a DEVICE pointer (memory the caller allocated
 *    on the GPU that is current when the call is made).  Tensors are
 *    row-major and contiguous.  bf16 values travel as their uint16_t bit
 *    patterns.  `stream` is a hipStream_t passed as void* (NULL = the
 *    default stream).
 *  * Ownership: the caller owns and allocates everything (pools, scales,
 *    tables, lengths, partials, outputs).  The library allocates no device
 *    memory, frees nothing and never synchronises; each call only enqueues
 *    kernels on `stream` and returns.  The balanced schedules read the
 *    current device's compute-unit count and kernel occupancy once per
 *    device and configuration and keep them in a small host-side table
 *    (the only state between calls).  Calls are thread-safe.
 *  * Errors: scalar arguments and pointer alignment are checked on the
 *    host before anything is launched.  A bad argument returns
 *    PKV_EINVAL, a shape outside the compiled kernel set returns
 *    PKV_EUNSUPPORTED; nothing is launched in either case.  PKV_ELAUNCH
 *    reports a launch failure (hipGetLastError).  Device-resident CONTENTS
 *    (table entries, lengths) are preconditions, as for an OS page table,
 *    and are not checked by the kernels: see "Table preconditions".
 *
 * Cache layout ([B] "PagedAttention": fixed-size physical blocks, any
 * free block serves any sequence)
 * ------------------------------------------------------------------
 *  k_cache, v_cache : [num_blocks, block_size, Hkv, D]
 *      kv_dtype PKV_BF16        : uint16_t bf16 bits
 *      kv_dtype PKV_FP8_E4M3*   : uint8_t OCP E4M3FN codes (max finite 448,
 *                                 0x7F/0xFF NaN, no infinities)
 *      kv_dtype PKV_INT8        : uint8_t codes u in [0, 255]
 *  k_scale, v_scale (NULL for bf16), dequantise on read ([B] "FP8 KV
 *  cache": a scale factor per tensor or per head; [B] "INT8 KV cache":
 *  symmetric or asymmetric with a scale and a zero point):
 *      PKV_FP8_E4M3            [num_blocks, Hkv] : decode(c) * scale[p, h]
 *      PKV_FP8_E4M3_PER_HEAD   [Hkv]             : decode(c) * scale[h]
 *      PKV_FP8_E4M3_PER_TENSOR [1]               : decode(c) * scale[0]
 *      PKV_INT8                [num_blocks, Hkv, 2] (scale, zero point)
 *                                                : scale * (u - zero point);
 *          zero point integer-valued in [0, 255]; symmetric quantisation
 *          is zero point 128.
 *  Writes (append, write) encode x as E4M3FN(x / scale) (round to nearest
 *  even, saturate to +-448) or clamp(rint(x / scale) + zero point, 0, 255)
 *  (NaN -> 0), with a correctly rounded binary32 division; the scales are
 *  the caller's (values outside their range saturate).
 *  block_tables : [B, max_blocks] int32.  Logical block j of sequence b
 *      lives in physical block block_tables[b, j]; token t of sequence b
 *      is slot t % block_size of logical block t / block_size
 *      ([B] "PagedAttention": the block table maps logical blocks to
 *      physical ones).  Several tables may name the same physical block
 *      (shared prefixes, [B] "PagedAttention" / [A] prefix caching).
 *  context_lens : [B] int32, the number of tokens of each sequence,
 *      INCLUDING the token appended in the current decode step ([B] "What
 *      the KV Cache Stores and Why": a step computes K, V for the new
 *      token only and then attends the new query over every cached token).
 *
 * Table preconditions (not checked on the device)
 * -----------------------------------------------
 *  0 <= context_lens[b] <= max_blocks * block_size;
 *  0 <= block_tables[b, j] < num_blocks for j < ceil(context_lens[b] / block_size);
 *  entries past that are never read;
 *  paged_kv_append must not target a block that another table also names.
 *
 * Cross-layer sharing ([A] "What is cross-layer KV sharing"): the layer ->
 * group "shared-with" pointer is the caller passing the group's cache and
 * scale pointers to the per-layer call; the kernels need nothing else.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
    PKV_OK = 0,
    PKV_EINVAL = -1,        /* bad scalar, null or misaligned pointer      */
    PKV_EUNSUPPORTED = -2,  /* shape outside the compiled kernel set       */
    PKV_ELAUNCH = -3,       /* the HIP runtime reported a launch failure   */
    PKV_ENOSPACE = -4,      /* block manager: not enough free or evictable
                               blocks (nothing changed)                    */
    PKV_ENOMEM = -5         /* block manager: host allocation failed       */
};

enum pkv_dtype {
    PKV_BF16 = 0,
    PKV_FP8_E4M3 = 1,           /* OCP E4M3FN, per-(block, kv head) fp32 scale */
    PKV_FP8_E4M3_PER_HEAD = 2,  /* OCP E4M3FN, one scale per kv head           */
    PKV_FP8_E4M3_PER_TENSOR = 3,/* OCP E4M3FN, one scale for the whole cache    */
    PKV_INT8 = 4                /* uint8 codes, per-(block, kv head) scale and
                                   zero point                                   */
};

/* Supported shapes of this build: D in {64, 128}; block_size in {16, 32};
 * 1 <= Hq / Hkv <= 16; Hq % Hkv == 0. */

/*
 * paged_kv_append -- write the decode step's new K and V rows into the cache.
 *
 * [B] "What the KV Cache Stores and Why": each generation step computes
 * K and V for the new token only and stores them beside the cached ones.
 * For each sequence b with T = context_lens[b] > 0 the new token is at
 * logical position t = T - 1, so for every kv head h
 *     k_cache[block_tables[b, t / block_size], t % block_size, h, :] = k_new[b, h, :]
 * (likewise V).  Sequences with T == 0 are skipped.
 *
 * PKV_BF16: the bf16 bits are copied unchanged.
 * PKV_FP8_E4M3 ([B] "FP8 KV cache": quantise on write with a scale):
 *     code = E4M3FN_rne_satfinite( float(x) / scale[p, h] )
 *     using the block's existing scale (binary32 division, correctly
 *     rounded; ties to even; magnitudes beyond 448 saturate to +-448;
 *     NaN -> 0x7F).
 *
 *  k_new, v_new : [B, Hkv, D] bf16 bits (device)
 *  k_cache, v_cache, k_scale, v_scale, block_tables, context_lens : as above
 *  Every byte other than the B x Hkv new rows is left unchanged.
 *  Alignment: k_new/v_new/caches 16 bytes (8 for fp8 caches).
 */
int paged_kv_append(const uint16_t* k_new, const uint16_t* v_new,
                    void* k_cache, void* v_cache,
                    const float* k_scale, const float* v_scale,
                    const int32_t* block_tables, int32_t max_blocks,
                    const int32_t* context_lens,
                    int32_t B, int32_t Hkv, int32_t D, int32_t block_size,
                    int32_t num_blocks, int32_t kv_dtype, void* stream);

/*
 * paged_decode_attention -- one query token per sequence attends over all of
 * its cached K/V, gathered through the block table.
 *
 * [B] "What the KV Cache Stores and Why" (attend the new Q over every
 * cached K, V), [B] "PagedAttention" (the kernel locates each token's block
 * through the table), [B] "Attention Variants" (grouped-query heads: query
 * head hq reads kv head hq / (Hq / Hkv)).  The attention itself is
 * standard softmax attention with an explicit scale (the pages do not
 * spell it out):
 *     s_t   = scale * dot(query[b, hq, :], K_t)            t in [0, T_b)
 *     out   = sum_t softmax(s)_t * V_t
 *     lse   = ln sum_t exp(s_t)
 * computed in fp32 from bf16 (or dequantised fp8) inputs.
 *
 *  query : [B, Hq, D] bf16 bits
 *  scale : softmax scale, usually 1/sqrt(D)
 *
 * split_tokens == 0 (single pass): writes out [B, Hq, D] float and, when
 *     lse_out is non-NULL, lse_out [B, Hq] float.  partial_out, partial_lse
 *     and max_splits are ignored.  A sequence with T == 0 gets out = 0,
 *     lse = -inf.
 * split_tokens > 0 (split context, a multiple of block_size): the context
 *     of sequence b is cut into ceil(T_b / split_tokens) consecutive
 *     ranges [s*S, min(T_b, (s+1)*S)), each attended independently (long
 *     contexts are a bandwidth problem, [B] "Two Costs: Capacity and
 *     Bandwidth"; independent ranges keep every compute unit streaming).
 *     Writes the normalised partial outputs and their natural-log lse:
 *         partial_out [B, Hq, max_splits, D] float
 *         partial_lse [B, Hq, max_splits]    float
 *     for s < ceil(T_b / S); other entries are untouched.  out and lse_out
 *     are NOT written: combine the partials with split_context_reduce on
 *     the same stream.  Requires max_splits >= ceil(max_b T_b / S) (a
 *     precondition on the device-resident lengths, not checked: tokens past
 *     max_splits * S would not be attended, the fused append would not
 *     write such a sequence's row, and split_context_reduce reads at most
 *     max_splits slots of a row).
 *
 *  Alignment: query, caches, out and partial_out 16 bytes.
 */
int paged_decode_attention(const uint16_t* query,
                           const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                           int32_t block_size, int32_t num_blocks,
                           int32_t kv_dtype, float scale,
                           int32_t split_tokens,
                           float* out,
                           float* partial_out, float* partial_lse,
                           int32_t max_splits, float* lse_out, void* stream);

/*
 * split_context_reduce -- combine split-context partials into the final
 * output with the log-sum-exp identity (not on the pages; it is the exact
 * rule for softmax attention over disjoint key sets):
 *     M   = max_s lse_s,   w_s = exp(lse_s - M)
 *     out = sum_s w_s * o_s / sum_s w_s,   lse = M + ln sum_s w_s
 * over the ceil(T_b / split_tokens) live splits of each sequence.  A split
 * with lse_s = -inf (no tokens) carries no weight; if every split is
 * -inf the result is out = 0, lse = -inf.
 *
 *  partial_out [B, Hq, max_splits, D], partial_lse [B, Hq, max_splits] float
 *  out [B, Hq, D] float; lse_out [B, Hq] float or NULL.
 *  Alignment: partial_out and out 16 bytes.
 */
int split_context_reduce(const float* partial_out, const float* partial_lse,
                         const int32_t* context_lens,
                         int32_t B, int32_t Hq, int32_t D,
                         int32_t split_tokens, int32_t max_splits,
                         float* out, float* lse_out, void* stream);

/*
 * paged_decode_attention_balanced -- the same operation as the single-pass
 * mode of paged_decode_attention (same arguments, same out / lse_out),
 * scheduled for ragged batches.
 *
 * Decode time is the bytes streamed ([B] "Two Costs: Capacity and
 * Bandwidth"); with ragged context lengths ([B] "Continuous Batching":
 * sequences of every length share one decode iteration) a fixed
 * one-unit-per-(sequence, head) grid leaves most compute units idle
 * while the longest sequences finish.  Here the 32-token tiles of all
 * (sequence, kv head) pairs form one list that is cut into equal ranges,
 * one per launched work-group (a group of kv heads walks a range
 * together; every group starts at once: one group per compute unit for
 * four-head groups of bf16 / fp8 caches, as many as fit otherwise); a
 * pair cut by range boundaries is finished by a log-sum-exp merge of its
 * pieces (second launch, same stream).
 *
 *  workspace       : device scratch of at least workspace_bytes, 16-byte
 *                    aligned, owned by the caller; its contents on entry are
 *                    irrelevant and on return unspecified.  Calls that share
 *                    one workspace must be ordered on one stream.
 *  workspace_bytes : >= paged_decode_workspace_size(Hq, Hkv, D, block_size,
 *                    kv_dtype) for the device current at the call.
 *  out, lse_out    : as in single-pass paged_decode_attention (T == 0 gives
 *                    out = 0, lse = -inf).
 *  Returns PKV_EINVAL if the workspace is too small; PKV_EUNSUPPORTED if
 *  max_blocks * block_size exceeds 2^25 tokens.
 */
int paged_decode_attention_balanced(const uint16_t* query,
                                    const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* block_tables, int32_t max_blocks,
                                    const int32_t* context_lens,
                                    int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t block_size, int32_t num_blocks,
                                    int32_t kv_dtype, float scale,
                                    void* workspace, int64_t workspace_bytes,
                                    float* out, float* lse_out, void* stream);

/*
 * paged_append_decode_attention, paged_append_decode_attention_balanced --
 * one decode step's append and attention in one launch: exactly
 * paged_kv_append(k_new, v_new, ...) followed on the same stream by
 * paged_decode_attention / paged_decode_attention_balanced with the same
 * arguments ([B] "What the KV Cache Stores and Why": the step stores the
 * new token's K and V, then its query attends over every cached token,
 * the new one included).  The wave that attends a sequence's last
 * position writes that position's row first, so the caches are both
 * written and read by the call.
 *
 *  k_new, v_new   : [B, Hkv, D] bf16 bits (device), 16-byte aligned, as in
 *                   paged_kv_append (same encoding for 1-byte formats, with
 *                   the block's existing scale).
 *  k_cache, v_cache : written at slot T_b - 1 of every sequence with
 *                   T_b > 0, read everywhere else as in the attention call.
 *  Other arguments, outputs, alignment and errors as in the attention call
 *  (PKV_EINVAL also for a missing k_new / v_new).  The written slot must
 *  belong to its sequence alone: a physical block shared with another
 *  sequence of the batch (prefix sharing) is copied before its first
 *  append (copy-on-write), as for paged_kv_append.
 */
int paged_append_decode_attention(const uint16_t* query,
                                  const uint16_t* k_new, const uint16_t* v_new,
                                  void* k_cache, void* v_cache,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* block_tables, int32_t max_blocks,
                                  const int32_t* context_lens,
                                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t block_size, int32_t num_blocks,
                                  int32_t kv_dtype, float scale,
                                  int32_t split_tokens,
                                  float* out,
                                  float* partial_out, float* partial_lse,
                                  int32_t max_splits, float* lse_out, void* stream);

int paged_append_decode_attention_balanced(const uint16_t* query,
                                           const uint16_t* k_new, const uint16_t* v_new,
                                           void* k_cache, void* v_cache,
                                           const float* k_scale, const float* v_scale,
                                           const int32_t* block_tables, int32_t max_blocks,
                                           const int32_t* context_lens,
                                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                           int32_t block_size, int32_t num_blocks,
                                           int32_t kv_dtype, float scale,
                                           void* workspace, int64_t workspace_bytes,
                                           float* out, float* lse_out, void* stream);

/*
 * paged_decode_attention_balanced_noalloc -- paged_decode_attention_balanced
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results without workspace / workspace_bytes.  Its workspace
 * is a static device array inside the library, 18 MiB per GPU, held from
 * the library's first use on that GPU until the process ends (its contents
 * on entry do not matter, as for a caller-owned workspace).  Nothing is
 * allocated or freed by any call.  All calls on one GPU share that GPU's
 * array: calls that may overlap on one GPU (different streams, threads
 * without ordering) race and give wrong results; order them on one stream.
 *  Returns PKV_EUNSUPPORTED when the workspace of these shapes on this
 *  device (paged_decode_workspace_size) exceeds 18 MiB, PKV_ELAUNCH if the
 *  array's device address cannot be obtained, otherwise as
 *  paged_decode_attention_balanced.
 */
int paged_decode_attention_balanced_noalloc(const uint16_t* query,
                                            const void* k_cache, const void* v_cache,
                                            const float* k_scale, const float* v_scale,
                                            const int32_t* block_tables, int32_t max_blocks,
                                            const int32_t* context_lens,
                                            int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t block_size, int32_t num_blocks,
                                            int32_t kv_dtype, float scale,
                                            float* out, float* lse_out, void* stream);

/*
 * Bytes of workspace paged_decode_attention_balanced needs for these
 * head counts and cache format on the current device (it depends on the
 * device's compute-unit count), or a negative pkv_status.  Independent of
 * the batch and of the context lengths.
 */
int64_t paged_decode_workspace_size(int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t block_size, int32_t kv_dtype);

/*
 * ---------------------------------------------------------------------
 * Several new tokens per sequence in one step: a chunk of a long prompt
 * ([B] "Continuous Batching": chunked prefill feeds a prompt in pieces
 * interleaved with decodes) or the draft tokens a target model verifies
 * in one pass ([A] "How does speculative decoding interact with KV-cache
 * compression").  Sequence b brings q_b = query_start[b+1] -
 * query_start[b] new tokens, its LAST q_b positions: row query_start[b] + i
 * is position p = T_b - q_b + i, where T_b = context_lens[b] counts the new
 * tokens.  Rows are laid out [total_rows, H, D] (H = Hkv for K/V rows, Hq
 * for queries and outputs).
 *
 * Device-side preconditions (not checked by the kernels): query_start is
 * non-decreasing with 0 <= q_b <= T_b and query_start[B] <= total_rows;
 * the table covers ceil(T_b / block_size) blocks of each sequence.
 * ---------------------------------------------------------------------
 */

/*
 * paged_kv_write -- store each sequence's q_b new K/V rows at positions
 * T_b - q_b .. T_b - 1 (the single-token append is q_b = 1).
 *
 *  k_rows, v_rows : [total_rows, Hkv, D] bf16 bits (device, 16-byte aligned).
 *  query_start    : [B + 1] int32 row offsets (device).
 *  max_query_len  : >= max_b q_b (host); sizes the launch, rows past q_b of
 *                   a sequence are never read.
 *  Other arguments, fp8 encoding and errors as paged_kv_append; B > 65535
 *  or max_query_len > 2^25 is PKV_EUNSUPPORTED.  fp8 writes use the block's
 *  existing scale and saturate to +-448.
 */
int paged_kv_write(const uint16_t* k_rows, const uint16_t* v_rows,
                   const int32_t* query_start,
                   void* k_cache, void* v_cache,
                   const float* k_scale, const float* v_scale,
                   const int32_t* block_tables, int32_t max_blocks,
                   const int32_t* context_lens,
                   int32_t B, int32_t max_query_len, int32_t Hkv, int32_t D,
                   int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                   void* stream);

/*
 * paged_multiquery_attention -- causal attention of every new token: row
 * query_start[b] + i (position p = T_b - q_b + i) attends over tokens
 * [0, p] of sequence b, query head hq through kv head hq / (Hq / Hkv), with
 * the same scaled softmax as paged_decode_attention.  Call after
 * paged_kv_write of the same rows.  Scheduled like
 * paged_decode_attention_balanced: every sequence's tokens are streamed
 * once per kv head while its q_b * G (new row, query head) pairs are at
 * most 32, once per 32 pairs up to 128; when max_query_len * G exceeds 128
 * (prefill chunks) a work-group per 256 pairs stages each K/V tile in LDS
 * for all of them (the workspace is then unused).
 *
 *  query          : [total_rows, Hq, D] bf16 bits (device, 16-byte aligned).
 *  query_start    : [B + 1] int32 (device); total_rows, max_query_len host.
 *  workspace      : device scratch of >= workspace_bytes, 16-byte aligned,
 *                   caller-owned, contents on entry irrelevant; calls that
 *                   share one must be ordered on one stream.
 *  workspace_bytes: >= paged_multiquery_workspace_size(Hq, Hkv, D,
 *                   block_size, kv_dtype, max_query_len).
 *  out            : [total_rows, Hq, D] float; lse_out [total_rows, Hq]
 *                   float (natural log) or NULL.  Rows of no sequence are
 *                   untouched.
 *  Returns PKV_EINVAL for bad arguments or a small workspace,
 *  PKV_EUNSUPPORTED for shapes outside the kernel set (as the decode) or
 *  more than 2^25 tokens per sequence.
 */
int paged_multiquery_attention(const uint16_t* query, const int32_t* query_start,
                               int32_t total_rows, int32_t max_query_len,
                               const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int32_t max_blocks,
                               const int32_t* context_lens,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t block_size, int32_t num_blocks,
                               int32_t kv_dtype, float scale,
                               void* workspace, int64_t workspace_bytes,
                               float* out, float* lse_out, void* stream);

/*
 * Bytes of workspace paged_multiquery_attention needs on the current
 * device for these shapes and max_query_len, or a negative pkv_status.
 */
int64_t paged_multiquery_workspace_size(int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t block_size, int32_t kv_dtype,
                                        int32_t max_query_len);

/*
 * ---------------------------------------------------------------------
 * Whole-block moves ([C] "When the cache fills": preempting a sequence by
 * swapping its cache to host memory and back; "Offload"; [B]
 * "PagedAttention" block sharing, whose copy-on-write copies a block).
 * A block is block_size * Hkv * D * (2 bf16 | 1 fp8) contiguous bytes of
 * k_cache (and of v_cache), plus its Hkv scales of k_scale / v_scale for
 * fp8.  The block size in bytes must be a multiple of 16.  Buffers may be
 * device memory or pinned host memory the device can address
 * (hipHostMalloc); a move then streams over the host link.  Block id
 * CONTENTS are device-side preconditions: ids in [0, num_blocks), and for
 * copies no block both a source and a destination, no destination twice.
 * Returns PKV_EINVAL for null / misaligned (16 bytes) pointers or bad
 * sizes, PKV_EUNSUPPORTED if the block size in bytes is not a multiple of
 * 16; n == 0 is a no-op.
 * ---------------------------------------------------------------------
 */

/* k_out[i] = k_cache[block_ids[i]] (and V, and fp8 scales), i < n:
 * k_out, v_out [n, block_size, Hkv, D]; scale outputs [n, Hkv]. */
int paged_kv_gather_blocks(const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_ids, int32_t n,
                           int32_t block_size, int32_t Hkv, int32_t D,
                           int32_t num_blocks, int32_t kv_dtype,
                           void* k_out, void* v_out,
                           float* k_scale_out, float* v_scale_out, void* stream);

/* k_cache[block_ids[i]] = k_in[i] (and V, and fp8 scales), i < n. */
int paged_kv_scatter_blocks(const void* k_in, const void* v_in,
                            const float* k_scale_in, const float* v_scale_in,
                            const int32_t* block_ids, int32_t n,
                            int32_t block_size, int32_t Hkv, int32_t D,
                            int32_t num_blocks, int32_t kv_dtype,
                            void* k_cache, void* v_cache,
                            float* k_scale, float* v_scale, void* stream);

/* k_cache[dst_ids[i]] = k_cache[src_ids[i]] (and V, and fp8 scales). */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                         const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                         int32_t block_size, int32_t Hkv, int32_t D,
                         int32_t num_blocks, int32_t kv_dtype, void* stream);

/* Human-readable name of a pkv_status value (static storage). */
const char* pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
