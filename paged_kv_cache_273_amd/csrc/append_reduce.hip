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
// INT8 ([B] "INT8 KV cache"): code = clamp(rint(x / scale) + zero point,
// 0, 255) with a correctly rounded binary32 division and round-half-even;
// NaN gives 0.
__device__ __forceinline__ uint32_t f32_to_u8_zp(float x, float scale, float zp)
{
    const float y = x / scale;
    if (y != y)
        return 0u;
    const float v = __builtin_rintf(y) + zp;
    return (uint32_t)fminf(fmaxf(v, 0.f), 255.f);
}

// Scales (and int8 zero points) of one (block, kv head).
struct Quant {
    float ks, vs, kz, vz;
};

template <int KVF>
__device__ __forceinline__ Quant quant_of(const float* k_scale, const float* v_scale, int p,
                                          int h, int sc_blk, int sc_head)
{
    Quant q = {1.f, 1.f, 0.f, 0.f};
    if (KVF) {
        const size_t i = (size_t)p * sc_blk + (size_t)h * sc_head;
        q.ks = k_scale[i];
        q.vs = v_scale[i];
        if (KVF == 2) {
            q.kz = k_scale[i + 1];
            q.vz = v_scale[i + 1];
        }
    }
    return q;
}

// Moves 8 elements (16 bytes of bf16 input) of one K row and one V row
// into the cache at element offset dst, encoding for 1-byte formats.
template <int KVF>
__device__ __forceinline__ void store8(const uint16_t* k_src, const uint16_t* v_src,
                                       void* k_cache, void* v_cache, size_t dst, Quant q)
{
    const u32x4 kx = *(const u32x4*)k_src;
    const u32x4 vx = *(const u32x4*)v_src;
    if (!KVF) {
        *(u32x4*)((uint16_t*)k_cache + dst) = kx;
        *(u32x4*)((uint16_t*)v_cache + dst) = vx;
        return;
    }
    u32x2 kq = {0u, 0u}, vq = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float kf = bf16_bits_to_f32((kx[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
        const float vf = bf16_bits_to_f32((vx[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
        uint32_t kc, vc;
        if (KVF == 1) {
            kc = f32_to_e4m3_sat(kf / q.ks);
            vc = f32_to_e4m3_sat(vf / q.vs);
        } else {
            kc = f32_to_u8_zp(kf, q.ks, q.kz);
            vc = f32_to_u8_zp(vf, q.vs, q.vz);
        }
        kq[i / 4] |= kc << (8 * (i & 3));
        vq[i / 4] |= vc << (8 * (i & 3));
    }
    *(u32x2*)((uint8_t*)k_cache + dst) = kq;
    *(u32x2*)((uint8_t*)v_cache + dst) = vq;
}

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
// One 256-thread work-group per (b, hq).  Threads first take the live
// splits' lse values (M = max, w_s = exp(lse_s - M), W = sum w_s) and park
// w_s in LDS; then thread (group g, column c) sums w_s * o_s over the
// splits s = g, g + NG, ... for four output elements, four splits' loads
// at a time; the NG partial sums meet in LDS.
constexpr int kReduceThreads = 256;

__device__ __forceinline__ float block_reduce(float v, float* scratch, bool is_max)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();
    if (lane == 0)
        scratch[wave] = v;
    __syncthreads();
    float r = scratch[0];
    for (int i = 1; i < kReduceThreads / kWave; ++i)
        r = is_max ? fmaxf(r, scratch[i]) : r + scratch[i];
    return r;
}

__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(ReduceArgs a)
{
    extern __shared__ f32x4 red[];               // [kReduceThreads] then weights
    float* w_lds = (float*)(red + kReduceThreads);
    float* scratch = (float*)red;
    const int row = blockIdx.x;                  // b * Hq + hq
    const int b = row / a.Hq;
    const int tid = threadIdx.x;
    const int T = a.context_lens[b];
    const int ns = T > 0 ? (T + a.split_tokens - 1) / a.split_tokens : 0;
    const float* pl = a.partial_lse + (size_t)row * a.max_splits;
    const float* po = a.partial_out + (size_t)row * a.max_splits * a.D;
    float* o = a.out + (size_t)row * a.D;

    float m = -__builtin_inff();
    for (int s = tid; s < ns; s += kReduceThreads)
        m = fmaxf(m, pl[s]);
    m = block_reduce(m, scratch, true);
    if (m == -__builtin_inff()) {
        for (int d = tid; d < a.D; d += kReduceThreads)
            o[d] = 0.f;
        if (a.lse_out && tid == 0)
            a.lse_out[row] = -__builtin_inff();
        return;
    }
    float wsum = 0.f;
    for (int s = tid; s < ns; s += kReduceThreads) {
        const float l = pl[s];
        const float w = (l == -__builtin_inff()) ? 0.f : __expf(l - m);
        w_lds[s] = w;
        wsum += w;
    }
    wsum = block_reduce(wsum, scratch, false);   // also orders the w_lds writes
    const int cols = a.D / 4;
    const int ng = kReduceThreads / cols;
    const int col = tid % cols;
    const int grp = tid / cols;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (grp < ng) {
        // four splits' loads in flight per step
        constexpr int kBatch = 4;
        for (int s0 = grp; s0 < ns; s0 += kBatch * ng) {
            f32x4 v[kBatch];
            float w[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int s = s0 + k * ng;
                w[k] = s < ns ? w_lds[s] : 0.f;
                v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (w[k] != 0.f)
                    v[k] = *(const f32x4*)(po + (size_t)s * a.D + 4 * col);
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                acc += w[k] * v[k];
        }
    }
    __syncthreads();
    red[tid] = acc;
    __syncthreads();
    if (tid < cols) {
        f32x4 t = red[tid];
        for (int g = 1; g < ng; ++g)
            t += red[g * cols + tid];
        const float inv = 1.0f / wsum;
        *(f32x4*)(o + 4 * tid) = t * inv;
    }
    if (a.lse_out && tid == 0)
        a.lse_out[row] = m + __logf(wsum);
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
    const size_t lds = kReduceThreads * sizeof(f32x4) + (size_t)a.max_splits * sizeof(float);
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)rows), dim3(kReduceThreads), lds, stream,
                       a);
    return hipGetLastError();
}

} // namespace pkv
