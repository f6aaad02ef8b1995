// append_reduce.hip -- the small kernels around paged decode attention:
//   * paged_kv_append: scatter the step's new K/V rows into their slots;
//   * paged_kv_write: the same for several new tokens per sequence;
//   * split_context_reduce: log-sum-exp merge of split-context partials.
//
// Pages cited:
//   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
//        Attention Variants, and the Bandwidth Wall"
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

// ---------------------------------------------------------------- append
// [B] "What the KV Cache Stores and Why": a decode step computes K and V for
// the new token only; it is stored at logical position T - 1 of its
// sequence, i.e. slot (T-1) % bs of the physical block the table names for
// logical block (T-1) / bs ([B] "PagedAttention").
// One thread moves 8 elements (16 bytes of bf16 input) of one (b, h) row.
// fp8 ([B] "FP8 KV cache"): code = E4M3FN(float(x) / scale) with a
// correctly rounded binary32 division; int8: see f32_to_u8_zp.
template <int KVF>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    const int per_row = a.D / 8;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long total = (long long)a.B * a.Hkv * per_row;
    if (gid >= total)
        return;
    const int c = (int)(gid % per_row);
    const int h = (int)((gid / per_row) % a.Hkv);
    const int b = (int)(gid / ((long long)per_row * a.Hkv));
    const int T = a.context_lens[b];
    if (T <= 0)
        return;
    const int t = T - 1;
    const int p = a.block_tables[(size_t)b * a.max_blocks + t / a.block_size];
    const int slot = t % a.block_size;
    const size_t src = ((size_t)b * a.Hkv + h) * a.D + 8 * c;
    const size_t dst = (((size_t)p * a.block_size + slot) * a.Hkv + h) * a.D + 8 * c;
    store8<KVF>(a.k_new + src, a.v_new + src, a.k_cache, a.v_cache, dst,
                quant_of<KVF>(a.k_scale, a.v_scale, p, h, a.sc_blk, a.sc_head));
}

// ---------------------------------------------------------------- write
// Several new tokens per sequence (a prefill chunk, [B] "Continuous
// Batching"; draft tokens under verification): row query_start[b] + i goes
// to position T_b - q_b + i.  Grid (x: rows i x heads x 8-element chunks
// up to max_query_len rows, y: sequence b); threads past q_b exit.
template <int KVF>
__global__ __launch_bounds__(256) void write_kernel(WriteArgs a)
{
    const int per_row = a.D / 8;
    const int b = blockIdx.y;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int row0 = a.query_start[b];
    const int q = a.query_start[b + 1] - row0;
    if (gid >= (long long)q * a.Hkv * per_row)
        return;
    const int c = (int)(gid % per_row);
    const int h = (int)((gid / per_row) % a.Hkv);
    const int i = (int)(gid / ((long long)per_row * a.Hkv));
    const int t = a.context_lens[b] - q + i;
    if (t < 0)
        return;                                  // more new rows than tokens
    const int p = a.block_tables[(size_t)b * a.max_blocks + t / a.block_size];
    const int slot = t % a.block_size;
    const size_t src = ((size_t)(row0 + i) * a.Hkv + h) * a.D + 8 * c;
    const size_t dst = (((size_t)p * a.block_size + slot) * a.Hkv + h) * a.D + 8 * c;
    store8<KVF>(a.k_rows + src, a.v_rows + src, a.k_cache, a.v_cache, dst,
                quant_of<KVF>(a.k_scale, a.v_scale, p, h, a.sc_blk, a.sc_head));
}

// ---------------------------------------------------------------- reduce
// One 256-thread work-group per (b, hq); thread (group g, column c) owns
// four output elements and the splits s = g, g + NG, ...  Each thread keeps
// a running log-sum-exp state over its own splits (max m, weight sum w,
// weighted sum of outputs), kBatch splits' lse values and outputs loaded
// at a time with no dependence between them, so a row of up to
// kBatch * NG splits costs one round trip to memory; the NG group states
// then meet in LDS (the log-sum-exp merge is exact whatever the grouping
// of the splits).
constexpr int kReduceThreads = 256;
constexpr int kReduceBatch = 8;

__global__ __launch_bounds__(kReduceThreads)
void reduce_kernel(const float* pre_out, const float* pre_lse, const int32_t* pre_lens,
                   int32_t pre_Hq, int32_t pre_split_tokens, int32_t pre_max_splits, ReduceArgs a)
{
    // the fields of the first loads, again as leading scalars preloaded in
    // SGPRs: the length load waits for no argument fetch
    a.partial_out = pre_out;
    a.partial_lse = pre_lse;
    a.context_lens = pre_lens;
    a.Hq = pre_Hq;
    a.split_tokens = pre_split_tokens;
    a.max_splits = pre_max_splits;
    __shared__ f32x4 acc_lds[kReduceThreads];
    __shared__ float m_lds[kReduceThreads];
    __shared__ float w_lds[kReduceThreads];
    const int row = blockIdx.x;                  // b * Hq + hq
    const int b = row / a.Hq;
    const int tid = threadIdx.x;
    const int T = a.context_lens[b];
    // splits of the row, never more than its max_splits slots (a context
    // beyond max_splits * split_tokens breaks the caller's precondition; its
    // tail was not attended, and no slot outside the row is read)
    const int ns = T > 0 ? min((T + a.split_tokens - 1) / a.split_tokens, a.max_splits) : 0;
    const float* pl = a.partial_lse + (size_t)row * a.max_splits;
    const float* po = a.partial_out + (size_t)row * a.max_splits * a.D;
    float* o = a.out + (size_t)row * a.D;
    const int cols = a.D / 4;                    // D % 4 == 0, D <= 1024
    const int ng = kReduceThreads / cols;        // >= 1; threads past ng * cols idle
    const int col = tid % cols;
    const int grp = tid / cols;
    constexpr float kNegInf = -__builtin_inff();

    float m = kNegInf, w = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = grp < ng ? grp : ns; s0 < ns; s0 += kReduceBatch * ng) {
        float l[kReduceBatch];
        f32x4 v[kReduceBatch];
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k) {
            const int s = s0 + k * ng;
            l[k] = kNegInf;
            v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s < ns) {
                l[k] = pl[s];
                v[k] = *(const f32x4*)(po + (size_t)s * a.D + 4 * col);
            }
        }
        float mb = m;
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k)
            mb = fmaxf(mb, l[k]);
        if (mb == kNegInf)
            continue;                            // nothing visible yet
        const float c = __expf(m - mb);          // m = -inf: 0
        acc *= c;
        w *= c;
#pragma unroll
        for (int k = 0; k < kReduceBatch; ++k) {
            if (l[k] == kNegInf)
                continue;                        // empty split (or not loaded)
            const float e = __expf(l[k] - mb);
            acc += e * v[k];
            w += e;
        }
        m = mb;
    }
    acc_lds[tid] = acc;
    m_lds[tid] = m;
    w_lds[tid] = w;
    __syncthreads();
    if (tid >= cols)
        return;
    float M = kNegInf;
    for (int g = 0; g < ng; ++g)
        M = fmaxf(M, m_lds[g * cols + tid]);
    if (M == kNegInf) {                          // empty sequence or no finite lse
        *(f32x4*)(o + 4 * tid) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.lse_out && tid == 0)
            a.lse_out[row] = kNegInf;
        return;
    }
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    for (int g = 0; g < ng; ++g) {
        const float mg = m_lds[g * cols + tid];
        if (mg == kNegInf)
            continue;
        const float e = __expf(mg - M);
        t += e * acc_lds[g * cols + tid];
        W += e * w_lds[g * cols + tid];
    }
    *(f32x4*)(o + 4 * tid) = t * (1.0f / W);
    if (a.lse_out && tid == 0)
        a.lse_out[row] = M + __logf(W);
}

} // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream)
{
    const long long total = (long long)a.B * a.Hkv * (a.D / 8);
    if (total <= 0)
        return hipSuccess;
    const long long blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    if (a.kv_dtype == 2)
        hipLaunchKernelGGL(append_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (a.kv_dtype == 1)
        hipLaunchKernelGGL(append_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(append_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_write(const WriteArgs& a, hipStream_t stream)
{
    const long long per_seq = (long long)a.max_query_len * a.Hkv * (a.D / 8);
    if (per_seq <= 0 || a.B <= 0)
        return hipSuccess;
    const long long blocks = (per_seq + 255) / 256;
    if (blocks > 0x7FFFFFFFLL || a.B > 65535)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks, (unsigned)a.B);
    if (a.kv_dtype == 2)
        hipLaunchKernelGGL(write_kernel<2>, grid, dim3(256), 0, stream, a);
    else if (a.kv_dtype == 1)
        hipLaunchKernelGGL(write_kernel<1>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(write_kernel<0>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream)
{
    const long long rows = (long long)a.B * a.Hq;
    if (rows <= 0)
        return hipSuccess;
    if (rows > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)rows), dim3(kReduceThreads), 0, stream,
                       a.partial_out, a.partial_lse, a.context_lens, a.Hq, a.split_tokens,
                       a.max_splits, a);
    return hipGetLastError();
}

} // namespace pkv
