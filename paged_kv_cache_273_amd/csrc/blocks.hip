// blocks.hip -- whole-block moves of the paged cache: gather blocks into a
// contiguous buffer (swap out / offload), scatter them back (swap in), and
// copy blocks inside the pool (copy-on-write of a shared block).
//
// Pages cited:
//   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
//        Attention Variants, and the Bandwidth Wall" -- "PagedAttention"
//        (block sharing)
//   [C] "KV-Cache Engineering: The Memory Wall of LLM Serving" -- "When the
//        cache fills" (preemption by swapping to host memory), "Offload"
//
// A block of a pool is block_size * Hkv * D * bytes contiguous bytes
// ([num_blocks, block_size, Hkv, D] layout), so a move is a copy of
// contiguous 16-byte chunks: work-group (x, kv) copies chunk x % cpb of
// block x / cpb of the K (kv = 0) or V (kv = 1) pool, 4 chunks of 16 KB
// per thread group in flight, non-temporal loads (each byte is read once).
// Either side may be host memory that the device can address (pinned,
// hipHostMalloc): the same kernel then streams over the host link.
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kMoveThreads = 256;
constexpr int kMoveUnroll = 4;
constexpr int kChunk = kMoveThreads * kMoveUnroll * 16;   // bytes per work-group

__global__ __launch_bounds__(kMoveThreads) void move_blocks_kernel(BlockMoveArgs a)
{
    const long long cpb = (a.block_bytes + kChunk - 1) / kChunk;
    const long long x = blockIdx.x;
    const int i = (int)(x / cpb);
    const long long c = x - (long long)i * cpb;
    const int kv = blockIdx.y;
    const long long sb = a.src_ids ? a.src_ids[i] : i;
    const long long db = a.dst_ids ? a.dst_ids[i] : i;
    const unsigned char* src = (kv ? a.src_v : a.src_k) + sb * a.block_bytes;
    unsigned char* dst = (kv ? a.dst_v : a.dst_k) + db * a.block_bytes;
    const long long base = c * kChunk + (long long)threadIdx.x * 16;
    u32x4 v[kMoveUnroll];
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
        const long long off = base + (long long)u * kMoveThreads * 16;
        if (off < a.block_bytes)
            v[u] = __builtin_nontemporal_load((const u32x4*)(src + off));
    }
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
        const long long off = base + (long long)u * kMoveThreads * 16;
        if (off < a.block_bytes)
            *(u32x4*)(dst + off) = v[u];
    }
    if (c == 0 && a.scale_count > 0) {
        const float* ss = kv ? a.src_vs : a.src_ks;
        float* ds = kv ? a.dst_vs : a.dst_ks;
        for (int h = threadIdx.x; h < a.scale_count; h += kMoveThreads)
            ds[db * a.scale_count + h] = ss[sb * a.scale_count + h];
    }
}

} // namespace

hipError_t launch_move_blocks(const BlockMoveArgs& a, hipStream_t stream)
{
    if (a.n <= 0)
        return hipSuccess;
    const long long cpb = (a.block_bytes + kChunk - 1) / kChunk;
    const long long groups = cpb * a.n;
    if (groups > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)groups, 2), dim3(kMoveThreads), 0,
                       stream, a);
    return hipGetLastError();
}

} // namespace pkv
