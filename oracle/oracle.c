/*
 * oracle.c -- CPU reference for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product
 * (the HIP library and its Python binding) never calls it, and this file
 * shares no header, helper, table or constant with the HIP sources.
 *
 * Plain, slow, obviously correct: every floating-point value is widened
 * exactly to double, scores and softmax are computed in double with a
 * two-pass max / sum (no online rescaling, no blocking, no fusion).
 *
 * Pages cited (by title and section):
 *   [A] "KV-Cache Engineering: Paged Attention, Prefix Cache,
 *        Disaggregation (2026)" -- FAQ page.
 *   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
 *        Attention Variants, and the Bandwidth Wall".
 *   [C] "KV-Cache Engineering: The Memory Wall of LLM Serving".
 *
 * Readings taken where the pages are silent (each is listed with the
 * others in the design notes):
 *   - attention is standard scaled dot-product softmax attention with an
 *     explicit scale; no mask beyond the context length;
 *   - query head hq uses kv head hq / (Hq/Hkv) (contiguous GQA groups);
 *   - context_lens[b] counts the token appended in the same decode step;
 *   - FP8 is OCP E4M3FN (bias 7, max finite 448, NaN = S.1111.111, no
 *     infinities), round-to-nearest-even, saturating to +-448;
 *   - split-context partials are normalised outputs plus natural-log
 *     log-sum-exp values; an empty split has lse = -inf and is ignored;
 *   - several new tokens of one sequence (a prefill chunk, or draft tokens
 *     under verification) are its last q_b positions; new token i sits at
 *     position T_b - q_b + i and attends causally over [0, that position];
 *     fp8 writes use the block's existing scale and saturate.
 *
 * Parity pins for every function live in tests/ (marked "not gpu").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* KV size arithmetic                                                 */
/* [B] "Cache size calculation": per-token bytes are twice (K and V)   */
/* the product of layers, kv heads, head dimension and element bytes.  */
/* [C] "Why the cache explodes": the total multiplies that by sequence */
/* length and batch.                                                   */
/* ------------------------------------------------------------------ */
int64_t orc_kv_bytes_per_token(int64_t layers, int64_t kv_heads,
                               int64_t head_dim, int64_t dtype_bytes)
{
    return 2 * layers * kv_heads * head_dim * dtype_bytes;
}

int64_t orc_kv_bytes_total(int64_t layers, int64_t kv_heads, int64_t head_dim,
                           int64_t seq_len, int64_t dtype_bytes, int64_t batch)
{
    return orc_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes)
           * seq_len * batch;
}

/* ------------------------------------------------------------------ */
/* Element formats                                                    */
/* ------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3FN decode, written from the format definition:
 * sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * is subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities.
 * [B] "Quantized KV Cache" / "FP8 KV cache" names the E4M3 format. */
double orc_e4m3_value(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static double code_value_table[0x7F];
static int code_value_table_ready = 0;

/* Value of a non-negative finite code, memoised from orc_e4m3_value. */
static double code_value(int code)
{
    if (!code_value_table_ready) {
        int c;
        for (c = 0; c < 0x7F; ++c)
            code_value_table[c] = orc_e4m3_value((uint8_t)c);
        code_value_table_ready = 1;
    }
    return code_value_table[code];
}

/* Nearest E4M3FN code to y: round to nearest, ties to the code with an
 * even mantissa, magnitudes above the largest finite value (448, code
 * 0x7E) saturate to it, NaN maps to 0x7F.  The non-negative codes
 * 0x00..0x7E are strictly increasing in value, so the two neighbours of
 * |y| are found by bisection over the codes themselves. */
uint8_t orc_e4m3_encode(float y)
{
    uint8_t sign;
    double a, dlo, dhi;
    int lo, hi, c;
    if (isnan(y))
        return 0x7F;
    sign = signbit(y) ? 0x80 : 0x00;
    a = fabs((double)y);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    lo = 0x00;          /* value 0   <= a */
    hi = 0x7E;          /* value 448 >  a */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (code_value(mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    dlo = a - code_value(lo);
    dhi = code_value(hi) - a;
    if (dlo < dhi)
        c = lo;
    else if (dhi < dlo)
        c = hi;
    else
        c = (lo & 1) == 0 ? lo : hi;
    return (uint8_t)(sign | c);
}

/* Quantise-on-write ([B] "FP8 KV cache": values are divided by a scale
 * factor and stored as FP8).  The division is one IEEE binary32
 * division of the widened bf16 value by the binary32 scale. */
uint8_t orc_e4m3_quantize(uint16_t x_bf16, float scale)
{
    float x = (float)orc_bf16_value(x_bf16);
    float y = x / scale;
    return orc_e4m3_encode(y);
}

/* ------------------------------------------------------------------ */
/* INT8 cache ([B] "INT8 KV cache": symmetric or asymmetric integer     */
/* quantisation with a scale and a zero point).  Codes are unsigned     */
/* bytes u in [0, 255] standing for scale * (u - zero_point); symmetric */
/* quantisation is zero_point = 128.  Encoding: y = x / scale as one    */
/* binary32 division, rounded to the nearest integer (ties to even),    */
/* plus the zero point, clamped to [0, 255]; NaN gives code 0.          */
/* ------------------------------------------------------------------ */
uint8_t orc_int8_quantize(uint16_t x_bf16, float scale, float zero_point)
{
    float x = (float)orc_bf16_value(x_bf16);
    float y = x / scale;
    double v;
    if (y != y)
        return 0;
    v = (double)rintf(y) + (double)zero_point;
    if (v < 0.0)
        v = 0.0;
    if (v > 255.0)
        v = 255.0;
    return (uint8_t)v;
}

/* ------------------------------------------------------------------ */
/* Paged addressing                                                   */
/* [B] "PagedAttention": logical block j of a sequence lives in the    */
/* physical block its block table names; a token at logical position t */
/* is slot t % block_size of logical block t / block_size.  Pool layout */
/* is [num_blocks, block_size, Hkv, D].                                */
/* ------------------------------------------------------------------ */
static int64_t pool_index(int32_t phys, int32_t slot, int32_t h, int32_t d,
                          int32_t bs, int32_t Hkv, int32_t D)
{
    return (((int64_t)phys * bs + slot) * Hkv + h) * D + d;
}

/* Cache formats (kv_dtype) and where an element's scale lives
 * ([B] "FP8 KV cache": a per-tensor or per-head scale; the per-(block,
 * head) scale is the finest of these; [B] "INT8 KV cache"):
 *   0  bf16 bits, no scale
 *   1  E4M3FN codes, scales[phys * Hkv + h]
 *   2  E4M3FN codes, scales[h]            (per kv head)
 *   3  E4M3FN codes, scales[0]            (per tensor)
 *   4  uint8 codes, (scale, zero point) = scales[2 (phys * Hkv + h)], [.. + 1] */
static int orc_valid_dtype(int32_t kv_dtype)
{
    return kv_dtype >= 0 && kv_dtype <= 4;
}

static int64_t scale_index(int32_t kv_dtype, int32_t phys, int32_t h, int32_t Hkv)
{
    switch (kv_dtype) {
    case 1: return (int64_t)phys * Hkv + h;
    case 2: return h;
    case 3: return 0;
    default: return 2 * ((int64_t)phys * Hkv + h);
    }
}

/* Dequantised (or widened) cache element (dequantise on read). */
static double cache_value(const void* cache, const float* scales, int32_t kv_dtype,
                          int32_t phys, int32_t slot, int32_t h, int32_t d,
                          int32_t bs, int32_t Hkv, int32_t D)
{
    int64_t i = pool_index(phys, slot, h, d, bs, Hkv, D);
    int64_t si;
    if (kv_dtype == 0)
        return orc_bf16_value(((const uint16_t*)cache)[i]);
    si = scale_index(kv_dtype, phys, h, Hkv);
    if (kv_dtype == 4)
        return (double)scales[si] * ((double)((const uint8_t*)cache)[i] - (double)scales[si + 1]);
    return orc_e4m3_value(((const uint8_t*)cache)[i]) * (double)scales[si];
}

/* Stores one bf16 value into a cache element of any format. */
static void store_value(void* cache, const float* scales, int32_t kv_dtype, int64_t dst,
                        uint16_t x, int32_t phys, int32_t h, int32_t Hkv)
{
    int64_t si;
    if (kv_dtype == 0) {
        ((uint16_t*)cache)[dst] = x;
        return;
    }
    si = scale_index(kv_dtype, phys, h, Hkv);
    if (kv_dtype == 4)
        ((uint8_t*)cache)[dst] = orc_int8_quantize(x, scales[si], scales[si + 1]);
    else
        ((uint8_t*)cache)[dst] = orc_e4m3_quantize(x, scales[si]);
}

/* Checks the preconditions a block table must meet before any kernel
 * reads it: every sequence fits its table row, and every table entry
 * that covers a live token names a block inside the pool.
 * Returns 0, or -(1 + b) for the first offending sequence b. */
int32_t orc_check_tables(const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t B,
                         int32_t block_size, int32_t num_blocks)
{
    int32_t b, j;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t nblk;
        if (T < 0 || (int64_t)T > (int64_t)max_blocks * block_size)
            return -(1 + b);
        nblk = (T + block_size - 1) / block_size;
        for (j = 0; j < nblk; ++j) {
            int32_t p = block_tables[(int64_t)b * max_blocks + j];
            if (p < 0 || p >= num_blocks)
                return -(1 + b);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Append: write the new token's K and V into its slot.               */
/* [B] "What the KV Cache Stores and Why": each step computes K, V for  */
/* the new token only and stores them beside the cached ones.  With     */
/* context_lens counting the new token, it goes to logical position     */
/* T - 1.  A sequence with T == 0 has nothing to append.               */
/* ------------------------------------------------------------------ */
void orc_append(const uint16_t* k_new, const uint16_t* v_new,
                void* k_cache, void* v_cache,
                const float* k_scale, const float* v_scale,
                const int32_t* block_tables, int32_t max_blocks,
                const int32_t* context_lens, int32_t B, int32_t Hkv, int32_t D,
                int32_t block_size, int32_t kv_dtype)
{
    int32_t b, h, d;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t t, phys, slot;
        if (T <= 0)
            continue;
        t = T - 1;
        phys = block_tables[(int64_t)b * max_blocks + t / block_size];
        slot = t % block_size;
        for (h = 0; h < Hkv; ++h) {
            for (d = 0; d < D; ++d) {
                int64_t src = ((int64_t)b * Hkv + h) * D + d;
                int64_t dst = pool_index(phys, slot, h, d, block_size, Hkv, D);
                store_value(k_cache, k_scale, kv_dtype, dst, k_new[src], phys, h, Hkv);
                store_value(v_cache, v_scale, kv_dtype, dst, v_new[src], phys, h, Hkv);
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Attention of one query head over a logical token range [t0, t1).    */
/* [B] "What the KV Cache Stores and Why": the new Q attends over every */
/* cached K, V.  Reading: s_t = scale * q . k_t, out = softmax(s) . V.  */
/* [B] "Attention Variants": query heads are partitioned into groups    */
/* that share one K/V head (GQA; MHA and MQA are the two extremes).     */
/* Returns lse = m + ln(sum exp(s_t - m)); an empty range gives out = 0 */
/* and lse = -inf.                                                       */
/* ------------------------------------------------------------------ */
double orc_attend_range(const uint16_t* query, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_tables, int32_t max_blocks,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                        int32_t kv_dtype, double scale,
                        int32_t b, int32_t hq, int32_t t0, int32_t t1, double* out)
{
    int32_t G = Hq / Hkv;
    int32_t h = hq / G;
    int32_t n = t1 - t0;
    int32_t i, d;
    double* q;
    double* s;
    double m, l, lse;

    for (d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n <= 0)
        return -INFINITY;

    q = (double*)malloc(sizeof(double) * (size_t)D);
    s = (double*)malloc(sizeof(double) * (size_t)n);
    for (d = 0; d < D; ++d)
        q[d] = orc_bf16_value(query[((int64_t)b * Hq + hq) * D + d]);

    /* pass 1: scores */
    for (i = 0; i < n; ++i) {
        int32_t t = t0 + i;
        int32_t phys = block_tables[(int64_t)b * max_blocks + t / block_size];
        int32_t slot = t % block_size;
        double dot = 0.0;
        for (d = 0; d < D; ++d)
            dot += q[d] * cache_value(k_cache, k_scale, kv_dtype, phys, slot, h, d,
                                      block_size, Hkv, D);
        s[i] = scale * dot;
    }
    m = s[0];
    for (i = 1; i < n; ++i)
        if (s[i] > m)
            m = s[i];

    /* pass 2: weights, normaliser, weighted sum of V */
    l = 0.0;
    for (i = 0; i < n; ++i) {
        int32_t t = t0 + i;
        int32_t phys = block_tables[(int64_t)b * max_blocks + t / block_size];
        int32_t slot = t % block_size;
        double w = exp(s[i] - m);
        l += w;
        for (d = 0; d < D; ++d)
            out[d] += w * cache_value(v_cache, v_scale, kv_dtype, phys, slot, h, d,
                                      block_size, Hkv, D);
    }
    for (d = 0; d < D; ++d)
        out[d] /= l;
    lse = m + log(l);
    free(q);
    free(s);
    return lse;
}

/* ------------------------------------------------------------------ */
/* Log-sum-exp merge of n partial results (split-context decode).      */
/* Not on the pages: the standard identity for combining softmax       */
/* attention over disjoint key sets.  With M = max lse_s,               */
/* w_s = exp(lse_s - M): out = sum w_s o_s / sum w_s,                   */
/* lse = M + ln sum w_s.  Parts with lse = -inf carry no weight; if all */
/* are -inf the result is out = 0, lse = -inf.                          */
/* ------------------------------------------------------------------ */
double orc_lse_merge(const double* o_parts, const double* lse_parts, int32_t n,
                     int32_t D, double* out)
{
    int32_t s, d;
    double M = -INFINITY, W = 0.0;
    for (d = 0; d < D; ++d)
        out[d] = 0.0;
    for (s = 0; s < n; ++s)
        if (lse_parts[s] > M)
            M = lse_parts[s];
    if (M == -INFINITY)
        return -INFINITY;
    for (s = 0; s < n; ++s) {
        double w;
        if (lse_parts[s] == -INFINITY)
            continue;
        w = exp(lse_parts[s] - M);
        W += w;
        for (d = 0; d < D; ++d)
            out[d] += w * o_parts[(int64_t)s * D + d];
    }
    for (d = 0; d < D; ++d)
        out[d] /= W;
    return M + log(W);
}

/* ------------------------------------------------------------------ */
/* Whole-batch attention.                                              */
/*   split_tokens == 0: out[b, hq, :] and lse[b, hq] over [0, T_b).     */
/*   split_tokens  > 0: split s covers [s*S, min(T_b, (s+1)*S)) for     */
/*     s < ceil(T_b / S); its normalised output and lse go to            */
/*     partial_out[b, hq, s, :] / partial_lse[b, hq, s] (when non-NULL)  */
/*     and out/lse receive the merge of the splits.  Entries for         */
/*     s >= ceil(T_b / S) are left untouched.                           */
/* Returns 0, or -1 on bad arguments.                                   */
/* ------------------------------------------------------------------ */
int32_t orc_paged_attention(const uint16_t* query, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t block_size, int32_t kv_dtype, double scale,
                            int32_t split_tokens, int32_t max_splits,
                            double* out, double* lse,
                            double* partial_out, double* partial_lse)
{
    int32_t b, hq;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || block_size <= 0
        || split_tokens < 0 || !orc_valid_dtype(kv_dtype))
        return -1;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t ns = 0;
        if (split_tokens > 0) {
            ns = (T + split_tokens - 1) / split_tokens;
            if (ns > max_splits)
                return -1;
        }
        for (hq = 0; hq < Hq; ++hq) {
            double* o = out + ((int64_t)b * Hq + hq) * D;
            double l;
            if (split_tokens == 0) {
                l = orc_attend_range(query, k_cache, v_cache, k_scale, v_scale,
                                     block_tables, max_blocks, Hq, Hkv, D, block_size,
                                     kv_dtype, scale, b, hq, 0, T, o);
            } else {
                double* po = (double*)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1) * D);
                double* pl = (double*)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
                int32_t s, d;
                for (s = 0; s < ns; ++s) {
                    int32_t t0 = s * split_tokens;
                    int32_t t1 = t0 + split_tokens < T ? t0 + split_tokens : T;
                    pl[s] = orc_attend_range(query, k_cache, v_cache, k_scale, v_scale,
                                             block_tables, max_blocks, Hq, Hkv, D,
                                             block_size, kv_dtype, scale, b, hq, t0, t1,
                                             po + (int64_t)s * D);
                    if (partial_out) {
                        double* dst = partial_out + (((int64_t)b * Hq + hq) * max_splits + s) * D;
                        for (d = 0; d < D; ++d)
                            dst[d] = po[(int64_t)s * D + d];
                    }
                    if (partial_lse)
                        partial_lse[((int64_t)b * Hq + hq) * max_splits + s] = pl[s];
                }
                l = orc_lse_merge(po, pl, ns, D, o);
                free(po);
                free(pl);
            }
            if (lse)
                lse[(int64_t)b * Hq + hq] = l;
        }
    }
    return 0;
}

/* Merge of binary32 partials laid out as the split kernels write them:
 * partial_out [B, Hq, max_splits, D], partial_lse [B, Hq, max_splits];
 * sequence b has ceil(T_b / split_tokens) live splits. */
int32_t orc_split_reduce(const float* partial_out, const float* partial_lse,
                         const int32_t* context_lens, int32_t B, int32_t Hq, int32_t D,
                         int32_t split_tokens, int32_t max_splits,
                         double* out, double* lse)
{
    int32_t b, hq, s, d;
    double* po;
    double* pl;
    if (split_tokens <= 0 || max_splits <= 0)
        return -1;
    po = (double*)malloc(sizeof(double) * (size_t)max_splits * D);
    pl = (double*)malloc(sizeof(double) * (size_t)max_splits);
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t ns = (T + split_tokens - 1) / split_tokens;
        if (ns > max_splits) {
            free(po);
            free(pl);
            return -1;
        }
        for (hq = 0; hq < Hq; ++hq) {
            int64_t row = (int64_t)b * Hq + hq;
            for (s = 0; s < ns; ++s) {
                pl[s] = (double)partial_lse[row * max_splits + s];
                for (d = 0; d < D; ++d)
                    po[(int64_t)s * D + d] = (double)partial_out[(row * max_splits + s) * D + d];
            }
            {
                double l = orc_lse_merge(po, pl, ns, D, out + row * D);
                if (lse)
                    lse[row] = l;
            }
        }
    }
    free(po);
    free(pl);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Several new tokens per sequence (chunked prefill, speculative verify). */
/* [B] "Continuous Batching": chunked prefill feeds a long prompt in      */
/* pieces of several tokens; [A] "How does speculative decoding interact  */
/* with KV-cache compression": the target verifies several draft tokens   */
/* at once.  Sequence b brings q_b = query_start[b+1] - query_start[b]     */
/* new tokens, the last q_b positions of its context_lens[b] tokens: row  */
/* query_start[b] + i is position p = T_b - q_b + i.  Rows are            */
/* [total_rows, H, D] with H = Hkv for K/V rows, Hq for queries/outputs.  */
/* ------------------------------------------------------------------ */

/* Writes the new tokens' K and V rows into their slots (the single-token
 * append is the case q_b = 1).  Returns 0, or -1 if some q_b > T_b. */
int32_t orc_write_tokens(const uint16_t* k_rows, const uint16_t* v_rows,
                         const int32_t* query_start, void* k_cache, void* v_cache,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t B, int32_t Hkv, int32_t D,
                         int32_t block_size, int32_t kv_dtype)
{
    int32_t b, i, h, d;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t q = query_start[b + 1] - query_start[b];
        if (q > T || q < 0)
            return -1;
        for (i = 0; i < q; ++i) {
            int64_t row = query_start[b] + i;
            int32_t t = T - q + i;
            int32_t phys = block_tables[(int64_t)b * max_blocks + t / block_size];
            int32_t slot = t % block_size;
            for (h = 0; h < Hkv; ++h)
                for (d = 0; d < D; ++d) {
                    int64_t src = (row * Hkv + h) * D + d;
                    int64_t dst = pool_index(phys, slot, h, d, block_size, Hkv, D);
                    store_value(k_cache, k_scale, kv_dtype, dst, k_rows[src], phys, h, Hkv);
                    store_value(v_cache, v_scale, kv_dtype, dst, v_rows[src], phys, h, Hkv);
                }
        }
    }
    return 0;
}

/* Causal attention of every new token: row query_start[b] + i (position
 * p = T_b - q_b + i) attends over tokens [0, p] of sequence b, each query
 * head through its kv head as in the single-token case.  out
 * [total_rows, Hq, D] and lse [total_rows, Hq].  Each row is the
 * single-query attention of that row over the first p + 1 tokens.
 * Returns 0, or -1 on bad arguments. */
int32_t orc_multiquery_attention(const uint16_t* query, const int32_t* query_start,
                                 const void* k_cache, const void* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t B, int32_t Hq,
                                 int32_t Hkv, int32_t D, int32_t block_size, int32_t kv_dtype,
                                 double scale, double* out, double* lse)
{
    int32_t b, i, hq;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || block_size <= 0
        || !orc_valid_dtype(kv_dtype))
        return -1;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t q = query_start[b + 1] - query_start[b];
        const int32_t* table_row = block_tables + (int64_t)b * max_blocks;
        if (q > T || q < 0)
            return -1;
        for (i = 0; i < q; ++i) {
            int64_t row = query_start[b] + i;
            int32_t p = T - q + i;
            /* the row as a one-sequence batch: query [1, Hq, D], table [1, max_blocks] */
            const uint16_t* qrow = query + row * Hq * D;
            for (hq = 0; hq < Hq; ++hq) {
                double l = orc_attend_range(qrow, k_cache, v_cache, k_scale, v_scale,
                                            table_row, max_blocks, Hq, Hkv, D, block_size,
                                            kv_dtype, scale, 0, hq, 0, p + 1,
                                            out + (row * Hq + hq) * D);
                if (lse)
                    lse[row * Hq + hq] = l;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Whole-block moves.  [C] "When the cache fills" (preempting a sequence by */
/* swapping its cache to host memory) and "Offload"; [A] anti-pattern (5)   */
/* (offloading inactive sessions to CPU memory); [B] "PagedAttention"       */
/* block sharing, whose copy-on-write needs a block copy.  A block is        */
/* block_bytes contiguous bytes of a pool (K or V codes, or one block's     */
/* scales).                                                                 */
/* ------------------------------------------------------------------ */

/* out[i] = pool[ids[i]] for i < n. */
void orc_gather_blocks(const void* pool, const int32_t* ids, int32_t n, int64_t block_bytes,
                       void* out)
{
    int32_t i;
    for (i = 0; i < n; ++i)
        memcpy((char*)out + (int64_t)i * block_bytes,
               (const char*)pool + (int64_t)ids[i] * block_bytes, (size_t)block_bytes);
}

/* pool[ids[i]] = in[i] for i < n. */
void orc_scatter_blocks(const void* in, const int32_t* ids, int32_t n, int64_t block_bytes,
                        void* pool)
{
    int32_t i;
    for (i = 0; i < n; ++i)
        memcpy((char*)pool + (int64_t)ids[i] * block_bytes,
               (const char*)in + (int64_t)i * block_bytes, (size_t)block_bytes);
}

/* pool[dst[i]] = pool[src[i]] for i < n (no block is both a source and a
 * destination). */
void orc_copy_blocks(void* pool, const int32_t* src, const int32_t* dst, int32_t n,
                     int64_t block_bytes)
{
    int32_t i;
    for (i = 0; i < n; ++i)
        memcpy((char*)pool + (int64_t)dst[i] * block_bytes,
               (const char*)pool + (int64_t)src[i] * block_bytes, (size_t)block_bytes);
}

/* ------------------------------------------------------------------ */
/* FP8 cache population (used to build fp8 test caches).               */
/* [B] "FP8 KV cache": a dynamic scale factor per head.  Reading: one    */
/* binary32 scale per (physical block, kv head), amax / 448 over the     */
/* block's live tokens, 1 when that amax is 0 or the block is unused.   */
/* A block's live-token count is the largest one any table gives it.    */
/* ------------------------------------------------------------------ */
void orc_fp8_block_scales(const uint16_t* src_bf16, const int32_t* block_tables,
                          int32_t max_blocks, const int32_t* context_lens, int32_t B,
                          int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                          float* scales)
{
    int32_t* live = (int32_t*)calloc((size_t)num_blocks, sizeof(int32_t));
    int32_t b, j, p, h, slot, d;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t nblk = (T + block_size - 1) / block_size;
        for (j = 0; j < nblk; ++j) {
            int32_t n = T - j * block_size;
            if (n > block_size)
                n = block_size;
            p = block_tables[(int64_t)b * max_blocks + j];
            if (n > live[p])
                live[p] = n;
        }
    }
    for (p = 0; p < num_blocks; ++p) {
        for (h = 0; h < Hkv; ++h) {
            double amax = 0.0;
            for (slot = 0; slot < live[p]; ++slot)
                for (d = 0; d < D; ++d) {
                    double v = fabs(orc_bf16_value(
                        src_bf16[pool_index(p, slot, h, d, block_size, Hkv, D)]));
                    if (v > amax)
                        amax = v;
                }
            scales[(int64_t)p * Hkv + h] = amax > 0.0 ? (float)amax / 448.0f : 1.0f;
        }
    }
    free(live);
}

/* Live slots of every physical block (the largest count any table gives
 * it); caller frees. */
static int32_t* live_slots(const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, int32_t B, int32_t block_size,
                           int32_t num_blocks)
{
    int32_t* live = (int32_t*)calloc((size_t)num_blocks, sizeof(int32_t));
    int32_t b, j;
    for (b = 0; b < B; ++b) {
        int32_t T = context_lens[b];
        int32_t nblk = (T + block_size - 1) / block_size;
        for (j = 0; j < nblk; ++j) {
            int32_t n = T - j * block_size;
            int32_t p = block_tables[(int64_t)b * max_blocks + j];
            if (n > block_size)
                n = block_size;
            if (n > live[p])
                live[p] = n;
        }
    }
    return live;
}

/* Per-kv-head (per_tensor = 0) or per-tensor (per_tensor = 1) E4M3 scales:
 * amax / 448 over the live tokens of every block (1 if amax = 0). */
void orc_fp8_wide_scales(const uint16_t* src_bf16, const int32_t* block_tables,
                         int32_t max_blocks, const int32_t* context_lens, int32_t B,
                         int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                         int32_t per_tensor, float* scales)
{
    int32_t* live = live_slots(block_tables, max_blocks, context_lens, B, block_size,
                               num_blocks);
    int32_t p, h, slot, d;
    double amax_t = 0.0;
    for (h = 0; h < Hkv; ++h) {
        double amax = 0.0;
        for (p = 0; p < num_blocks; ++p)
            for (slot = 0; slot < live[p]; ++slot)
                for (d = 0; d < D; ++d) {
                    double v = fabs(orc_bf16_value(
                        src_bf16[pool_index(p, slot, h, d, block_size, Hkv, D)]));
                    if (v > amax)
                        amax = v;
                }
        if (!per_tensor)
            scales[h] = amax > 0.0 ? (float)amax / 448.0f : 1.0f;
        if (amax > amax_t)
            amax_t = amax;
    }
    if (per_tensor)
        scales[0] = amax_t > 0.0 ? (float)amax_t / 448.0f : 1.0f;
    free(live);
}

/* INT8 (scale, zero point) pairs per (block, kv head) over the block's live
 * tokens.  Symmetric: scale = amax / 127, zero point 128.  Asymmetric:
 * scale = (max - min) / 255, zero point = rint(-min / scale) clamped to
 * [0, 255] (binary32 arithmetic).  A block or head with no spread gets
 * scale 1 (symmetric: amax = 0; asymmetric: max = min). */
void orc_int8_block_params(const uint16_t* src_bf16, const int32_t* block_tables,
                           int32_t max_blocks, const int32_t* context_lens, int32_t B,
                           int32_t Hkv, int32_t D, int32_t block_size, int32_t num_blocks,
                           int32_t symmetric, float* params)
{
    int32_t* live = live_slots(block_tables, max_blocks, context_lens, B, block_size,
                               num_blocks);
    int32_t p, h, slot, d;
    for (p = 0; p < num_blocks; ++p)
        for (h = 0; h < Hkv; ++h) {
            double lo = INFINITY, hi = -INFINITY, amax = 0.0;
            float sc, zp;
            for (slot = 0; slot < live[p]; ++slot)
                for (d = 0; d < D; ++d) {
                    double v = orc_bf16_value(
                        src_bf16[pool_index(p, slot, h, d, block_size, Hkv, D)]);
                    if (v != v)
                        continue;
                    if (v < lo)
                        lo = v;
                    if (v > hi)
                        hi = v;
                    if (fabs(v) > amax)
                        amax = fabs(v);
                }
            if (symmetric) {
                sc = amax > 0.0 ? (float)amax / 127.0f : 1.0f;
                zp = 128.0f;
            } else if (hi > lo) {
                float r;
                sc = ((float)hi - (float)lo) / 255.0f;
                r = rintf(-(float)lo / sc);
                zp = r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r);
            } else {
                sc = 1.0f;
                zp = 0.0f;
                if (lo == lo && lo < INFINITY) {
                    float r = rintf(-(float)lo);
                    zp = r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r);
                }
            }
            params[2 * ((int64_t)p * Hkv + h)] = sc;
            params[2 * ((int64_t)p * Hkv + h) + 1] = zp;
        }
    free(live);
}

/* Quantises a whole bf16 pool in any 1-byte format (kv_dtype 1-4). */
void orc_quantize_pool(const uint16_t* src_bf16, const float* scales, int32_t kv_dtype,
                       int32_t num_blocks, int32_t block_size, int32_t Hkv, int32_t D,
                       uint8_t* codes)
{
    int32_t p, slot, h, d;
    for (p = 0; p < num_blocks; ++p)
        for (slot = 0; slot < block_size; ++slot)
            for (h = 0; h < Hkv; ++h)
                for (d = 0; d < D; ++d) {
                    int64_t i = pool_index(p, slot, h, d, block_size, Hkv, D);
                    store_value(codes, scales, kv_dtype, i, src_bf16[i], p, h, Hkv);
                }
}

/* Quantises a whole bf16 pool [num_blocks, block_size, Hkv, D] with the
 * per-(block, kv head) scales.  NaN elements (poisoned slots) stay NaN. */
void orc_fp8_quantize_pool(const uint16_t* src_bf16, const float* scales,
                           int32_t num_blocks, int32_t block_size, int32_t Hkv, int32_t D,
                           uint8_t* codes)
{
    int32_t p, slot, h, d;
    for (p = 0; p < num_blocks; ++p)
        for (slot = 0; slot < block_size; ++slot)
            for (h = 0; h < Hkv; ++h) {
                float sc = scales[(int64_t)p * Hkv + h];
                for (d = 0; d < D; ++d) {
                    int64_t i = pool_index(p, slot, h, d, block_size, Hkv, D);
                    codes[i] = orc_e4m3_quantize(src_bf16[i], sc);
                }
            }
}
