// abi.hip -- the C ABI of libpagedkv.so (declared in include/pagedkv.h).
// Host-side argument checks, then one launch on the caller's stream.
// Nothing here allocates device memory, frees or synchronises (a small
// host-side table caches the resident work-group count per device and
// kernel configuration).
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

#include "../../include/pagedkv.h"
#include "../../include/pkv_probe.h"
#include "pkv_kernels.hpp"

namespace {

bool aligned(const void* p, uintptr_t n)
{
    return ((uintptr_t)p % n) == 0;
}

bool supported_d(int32_t D)
{
    return D == 64 || D == 128;
}

bool supported_bs(int32_t bs)
{
    return bs == 16 || bs == 32;
}

int launched(hipError_t e)
{
    return e == hipSuccess ? PKV_OK : PKV_ELAUNCH;
}

bool valid_dtype(int32_t kv_dtype)
{
    return kv_dtype >= PKV_BF16 && kv_dtype <= PKV_INT8;
}

bool one_byte(int32_t kv_dtype)
{
    return kv_dtype != PKV_BF16;
}

// Kernel format (0 bf16, 1 E4M3FN, 2 uint8 + zero point) and where the
// scale of (block p, kv head h) lives: k_scale[p * sc_blk + h * sc_head].
struct Fmt {
    int kvf, sc_blk, sc_head;
};

Fmt format_of(int32_t kv_dtype, int32_t Hkv)
{
    switch (kv_dtype) {
    case PKV_FP8_E4M3: return {1, Hkv, 1};
    case PKV_FP8_E4M3_PER_HEAD: return {1, 0, 1};
    case PKV_FP8_E4M3_PER_TENSOR: return {1, 0, 0};
    case PKV_INT8: return {2, 2 * Hkv, 2};
    default: return {0, 0, 0};
    }
}

// floats of one block's scale record that move with the block
int32_t scales_per_block(int32_t kv_dtype, int32_t Hkv)
{
    return kv_dtype == PKV_FP8_E4M3 ? Hkv : kv_dtype == PKV_INT8 ? 2 * Hkv : 0;
}


constexpr int32_t kMaxGroup = 16;     // query heads per kv head (one MFMA column tile)
// MI355X last-level (Infinity Cache / MALL) capacity.  A K+V pool that fits
// may be re-read from it by the next call; larger pools are streamed.
constexpr int64_t kMallBytes = (int64_t)256 << 20;
// per-sequence token bound of the balanced path (64-sequence tile sums stay in int32)
constexpr int64_t kMaxTokens = (int64_t)1 << 25;

// Load policy of the decode kernels: non-temporal (streaming) unless the
// whole K+V pool fits the MALL.  PKV_FORCE_LOAD_POLICY (0 = default
// policy, 1 = non-temporal) pins it at build time for measurements.
bool stream_kv_loads(int32_t num_blocks, int32_t block_size, int32_t Hkv, int32_t D,
                     int32_t kv_dtype)
{
#ifdef PKV_FORCE_LOAD_POLICY
    return PKV_FORCE_LOAD_POLICY != 0;
#else
    const int64_t esize = one_byte(kv_dtype) ? 1 : 2;
    const int64_t pool = 2 * (int64_t)num_blocks * block_size * Hkv * D * esize;
    return pool > kMallBytes;
#endif
}

} // namespace

// ------------------------------------------------------------- no allocation
// The allocation-free form of paged_decode_attention_balanced keeps its
// workspace in this file-scope device array (one copy per GPU, held until
// the process ends).  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address of
// each GPU's copy comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr int64_t kStaticScratchBytes = (int64_t)18 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of this device's scratch array, or null on failure.
void* device_scratch()
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> g(mu);
    if (addr[dev])
        return addr[dev];
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return nullptr;
    addr[dev] = p;
    return p;
}

} // namespace

extern "C" {

const char* pkv_status_string(int status)
{
    switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape";
    case PKV_ELAUNCH: return "kernel launch failed";
    case PKV_ENOSPACE: return "no free block";
    case PKV_ENOMEM: return "host allocation failed";
    default: return "unknown status";
    }
}

int paged_kv_append(const uint16_t* k_new, const uint16_t* v_new, void* k_cache, void* v_cache,
                    const float* k_scale, const float* v_scale, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* context_lens, int32_t B, int32_t Hkv,
                    int32_t D, int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                    void* stream)
{
    if (B < 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0 || max_blocks <= 0)
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size))
        return PKV_EUNSUPPORTED;
    if (B == 0)
        return PKV_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !context_lens)
        return PKV_EINVAL;
    const uintptr_t cache_align = one_byte(kv_dtype) ? 8 : 16;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, cache_align)
        || !aligned(v_cache, cache_align))
        return PKV_EINVAL;
    if (one_byte(kv_dtype) && (!k_scale || !v_scale))
        return PKV_EINVAL;
    pkv::AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks = max_blocks;
    a.B = B;
    a.Hkv = Hkv;
    a.D = D;
    a.block_size = block_size;
    const Fmt f = format_of(kv_dtype, Hkv);
    a.kv_dtype = f.kvf;
    a.sc_blk = f.sc_blk;
    a.sc_head = f.sc_head;
    return launched(pkv::launch_append(a, (hipStream_t)stream));
}

// Decode attention on the fixed partition; with k_new / v_new the launch
// also appends the step's new rows (paged_append_decode_attention).
static int decode_call(const uint16_t* query, const uint16_t* k_new, const uint16_t* v_new,
                       const void* k_cache, const void* v_cache, const float* k_scale,
                       const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                       float scale, int32_t split_tokens, float* out, float* partial_out,
                       float* partial_lse, int32_t max_splits, float* lse_out, void* stream)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0
        || max_blocks <= 0 || split_tokens < 0)
        return PKV_EINVAL;
    if (Hq % Hkv != 0 || !isfinite(scale))
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size) || Hq / Hkv > kMaxGroup)
        return PKV_EUNSUPPORTED;
    if (split_tokens > 0 && (split_tokens % block_size != 0 || max_splits <= 0))
        return PKV_EINVAL;
    if (B == 0)
        return PKV_OK;
    if (!query || !k_cache || !v_cache || !block_tables || !context_lens)
        return PKV_EINVAL;
    if (!aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
        return PKV_EINVAL;
    if (one_byte(kv_dtype) && (!k_scale || !v_scale))
        return PKV_EINVAL;
    if (k_new && (!v_new || !aligned(k_new, 16) || !aligned(v_new, 16)))
        return PKV_EINVAL;
    if (split_tokens == 0) {
        if (!out || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
            return PKV_EINVAL;
    } else {
        if (!partial_out || !partial_lse || !aligned(partial_out, 16))
            return PKV_EINVAL;
    }
    pkv::DecodeArgs a;
    a.query = query;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.lse_out = lse_out;
    a.partial_out = partial_out;
    a.partial_lse = partial_lse;
    a.query_start = nullptr;
    a.total_rows = 0;
    a.max_blocks = max_blocks;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.split_tokens = split_tokens;
    a.max_splits = split_tokens > 0 ? max_splits : 1;
    a.scale_log2 = scale * 1.4426950408889634f;
    const Fmt fmt = format_of(kv_dtype, Hkv);
    a.sc_blk = fmt.sc_blk;
    a.sc_head = fmt.sc_head;
    a.k_new = k_new;
    a.v_new = v_new;
    const bool nt = stream_kv_loads(num_blocks, block_size, Hkv, D, kv_dtype);
    return launched(pkv::launch_decode(a, D, block_size, fmt.kvf, nt, (hipStream_t)stream));
}

int paged_decode_attention(const uint16_t* query, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                           float scale, int32_t split_tokens, float* out, float* partial_out,
                           float* partial_lse, int32_t max_splits, float* lse_out, void* stream)
{
    return decode_call(query, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                       block_tables, max_blocks, context_lens, B, Hq, Hkv, D, block_size,
                       num_blocks, kv_dtype, scale, split_tokens, out, partial_out,
                       partial_lse, max_splits, lse_out, stream);
}

int paged_append_decode_attention(const uint16_t* query, const uint16_t* k_new,
                                  const uint16_t* v_new, void* k_cache, void* v_cache,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* block_tables, int32_t max_blocks,
                                  const int32_t* context_lens, int32_t B, int32_t Hq,
                                  int32_t Hkv, int32_t D, int32_t block_size,
                                  int32_t num_blocks, int32_t kv_dtype, float scale,
                                  int32_t split_tokens, float* out, float* partial_out,
                                  float* partial_lse, int32_t max_splits, float* lse_out,
                                  void* stream)
{
    if (B > 0 && (!k_new || !v_new))
        return PKV_EINVAL;
    return decode_call(query, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                       max_blocks, context_lens, B, Hq, Hkv, D, block_size, num_blocks,
                       kv_dtype, scale, split_tokens, out, partial_out, partial_lse,
                       max_splits, lse_out, stream);
}

// Work-groups of the balanced decode on the current device: exactly the
// number that can be resident at once, so every group starts immediately.
// Resident work-groups of one balanced-schedule kernel configuration on
// the current device (compute units x groups per CU), cached per device:
// the occupancy query is host work every call would otherwise repeat.
// nct = 0 selects the decode kernel, 1 or 2 the multi-query kernel.
static int resident_groups(int32_t Hkv, int32_t D, int32_t block_size, int32_t kv_dtype,
                           int nct)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    const int kvf = format_of(kv_dtype, Hkv).kvf;
    const int hg = pkv::balanced_head_group(Hkv, nct, kvf);
    const uint64_t key = ((((((uint64_t)dev * 256 + D) * 64 + block_size) * 4 + kvf) * 16 + hg)
                          * 4 + nct);
    static std::mutex mu;
    static std::unordered_map<uint64_t, int> cache;
    {
        std::lock_guard<std::mutex> g(mu);
        auto it = cache.find(key);
        if (it != cache.end())
            return it->second;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    int per_cu = nct == 0 ? pkv::balanced_groups_per_cu(D, block_size, kvf, hg)
                          : pkv::multiquery_groups_per_cu(D, block_size, kvf, hg, nct);
    if (pkv::balanced_one_group_per_cu(Hkv, nct, kvf) && per_cu > 1)
        per_cu = 1;
    const int n = cus * per_cu;
    if (n > 0) {
        std::lock_guard<std::mutex> g(mu);
        cache.emplace(key, n);
    }
    return n;
}

static int balanced_groups(int32_t Hkv, int32_t D, int32_t block_size, int32_t kv_dtype)
{
    return resident_groups(Hkv, D, block_size, kv_dtype, 0);
}

// Partial slots (2 per work-group) of rows_per_group rows, then the cut
// records at the next 16-byte boundary.
static int64_t schedule_bytes(int ngroups, int64_t rows_per_group, int32_t D)
{
    const int64_t rows = (int64_t)2 * ngroups * rows_per_group;
    const int64_t parts = rows * (D + 1) * (int64_t)sizeof(float);
    return (parts + 15) / 16 * 16 + (int64_t)ngroups * sizeof(pkv::CutRecord);
}

static void carve_workspace(pkv::BalanceArgs& ws, void* workspace, int64_t rows_per_group,
                            int32_t D)
{
    const int64_t rows = (int64_t)2 * ws.ngroups_launched * rows_per_group;
    ws.part_out = (float*)workspace;
    ws.part_lse = ws.part_out + (size_t)rows * D;
    const int64_t parts = rows * (D + 1) * (int64_t)sizeof(float);
    ws.cuts = (pkv::CutRecord*)((char*)workspace + (parts + 15) / 16 * 16);
}

static int64_t balanced_bytes(int ngroups, int32_t Hkv, int32_t G, int32_t D, int kvf)
{
    return schedule_bytes(ngroups, (int64_t)pkv::balanced_head_group(Hkv, 0, kvf) * G, D);
}

int64_t paged_decode_workspace_size(int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                    int32_t kv_dtype)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size) || Hq / Hkv > kMaxGroup)
        return PKV_EUNSUPPORTED;
    const int n = balanced_groups(Hkv, D, block_size, kv_dtype);
    if (n <= 0)
        return PKV_ELAUNCH;
    return balanced_bytes(n, Hkv, Hq / Hkv, D, format_of(kv_dtype, Hkv).kvf);
}

// Decode attention on the balanced schedule; with k_new / v_new the launch
// also appends the step's new rows (paged_append_decode_attention_balanced).
static int balanced_call(const uint16_t* query, const uint16_t* k_new, const uint16_t* v_new,
                         const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t D, int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                         float scale, void* workspace, int64_t workspace_bytes, float* out,
                         float* lse_out, void* stream)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0
        || max_blocks <= 0 || workspace_bytes < 0)
        return PKV_EINVAL;
    if (Hq % Hkv != 0 || !isfinite(scale))
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size) || Hq / Hkv > kMaxGroup)
        return PKV_EUNSUPPORTED;
    if ((int64_t)max_blocks * block_size > kMaxTokens)
        return PKV_EUNSUPPORTED;
    if (B == 0)
        return PKV_OK;
    if (!query || !k_cache || !v_cache || !block_tables || !context_lens || !out || !workspace)
        return PKV_EINVAL;
    if (!aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)
        || !aligned(out, 16) || !aligned(workspace, 16))
        return PKV_EINVAL;
    if (one_byte(kv_dtype) && (!k_scale || !v_scale))
        return PKV_EINVAL;
    if (k_new && (!v_new || !aligned(k_new, 16) || !aligned(v_new, 16)))
        return PKV_EINVAL;
    const int n = balanced_groups(Hkv, D, block_size, kv_dtype);
    if (n <= 0)
        return PKV_ELAUNCH;
    const int32_t G = Hq / Hkv;
    if (workspace_bytes < balanced_bytes(n, Hkv, G, D, format_of(kv_dtype, Hkv).kvf))
        return PKV_EINVAL;
    pkv::DecodeArgs a;
    a.query = query;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.lse_out = lse_out;
    a.partial_out = nullptr;
    a.partial_lse = nullptr;
    a.query_start = nullptr;
    a.total_rows = 0;
    a.max_blocks = max_blocks;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.split_tokens = 0;
    a.max_splits = 1;
    a.scale_log2 = scale * 1.4426950408889634f;
    const Fmt fmt = format_of(kv_dtype, Hkv);
    a.sc_blk = fmt.sc_blk;
    a.sc_head = fmt.sc_head;
    a.k_new = k_new;
    a.v_new = v_new;
    pkv::BalanceArgs ws;
    ws.head_group = pkv::balanced_head_group(Hkv, 0, fmt.kvf);
    // with four-head groups, the Hkv / 4 groups covering one token range
    // run side by side (neighbouring work-groups), so each 2 KB token row is
    // read whole at one time (measured ~1% faster than a range per group)
    ws.head_split = pkv::balanced_one_group_per_cu(Hkv, 0, fmt.kvf) ? Hkv / ws.head_group : 1;
    ws.ngroups_launched = n / ws.head_split * ws.head_split;
    carve_workspace(ws, workspace, (int64_t)ws.head_group * G, D);
    // range boundaries are computed in double precision: keep
    // (tiles of the call) * (groups launched) below 2^52
    const int64_t ngroups = Hkv / ws.head_group;
    const int64_t max_tiles = (int64_t)B * (((int64_t)max_blocks * block_size + 31) / 32) * ngroups;
    if (max_tiles * ((int64_t)n + 1) >= ((int64_t)1 << 52))
        return PKV_EUNSUPPORTED;
    const bool nt = stream_kv_loads(num_blocks, block_size, Hkv, D, kv_dtype);
    return launched(pkv::launch_decode_balanced(a, ws, D, block_size, fmt.kvf, nt,
                                                (hipStream_t)stream));
}

int paged_decode_attention_balanced(const uint16_t* query, const void* k_cache,
                                    const void* v_cache, const float* k_scale,
                                    const float* v_scale, const int32_t* block_tables,
                                    int32_t max_blocks, const int32_t* context_lens, int32_t B,
                                    int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                    int32_t num_blocks, int32_t kv_dtype, float scale,
                                    void* workspace, int64_t workspace_bytes, float* out,
                                    float* lse_out, void* stream)
{
    return balanced_call(query, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                         block_tables, max_blocks, context_lens, B, Hq, Hkv, D, block_size,
                         num_blocks, kv_dtype, scale, workspace, workspace_bytes, out, lse_out,
                         stream);
}

int paged_decode_attention_balanced_noalloc(const uint16_t* query, const void* k_cache,
                                            const void* v_cache, const float* k_scale,
                                            const float* v_scale, const int32_t* block_tables,
                                            int32_t max_blocks, const int32_t* context_lens,
                                            int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t block_size, int32_t num_blocks,
                                            int32_t kv_dtype, float scale, float* out,
                                            float* lse_out, void* stream)
{
    // the workspace this call needs must fit the static array
    const int64_t need = paged_decode_workspace_size(Hq, Hkv, D, block_size, kv_dtype);
    if (need < 0)
        return (int)need;
    if (need > kStaticScratchBytes)
        return PKV_EUNSUPPORTED;
    if (B == 0)
        return balanced_call(query, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                             block_tables, max_blocks, context_lens, B, Hq, Hkv, D, block_size,
                             num_blocks, kv_dtype, scale, nullptr, 0, out, lse_out, stream);
    void* ws = device_scratch();
    if (!ws)
        return PKV_ELAUNCH;
    return balanced_call(query, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                         block_tables, max_blocks, context_lens, B, Hq, Hkv, D, block_size,
                         num_blocks, kv_dtype, scale, ws, kStaticScratchBytes, out, lse_out,
                         stream);
}

int paged_append_decode_attention_balanced(const uint16_t* query, const uint16_t* k_new,
                                           const uint16_t* v_new, void* k_cache,
                                           void* v_cache, const float* k_scale,
                                           const float* v_scale, const int32_t* block_tables,
                                           int32_t max_blocks, const int32_t* context_lens,
                                           int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                           int32_t block_size, int32_t num_blocks,
                                           int32_t kv_dtype, float scale, void* workspace,
                                           int64_t workspace_bytes, float* out, float* lse_out,
                                           void* stream)
{
    if (B > 0 && (!k_new || !v_new))
        return PKV_EINVAL;
    return balanced_call(query, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                         block_tables, max_blocks, context_lens, B, Hq, Hkv, D, block_size,
                         num_blocks, kv_dtype, scale, workspace, workspace_bytes, out, lse_out,
                         stream);
}

int paged_kv_write(const uint16_t* k_rows, const uint16_t* v_rows, const int32_t* query_start,
                   void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
                   const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                   int32_t B, int32_t max_query_len, int32_t Hkv, int32_t D, int32_t block_size,
                   int32_t num_blocks, int32_t kv_dtype, void* stream)
{
    if (B < 0 || max_query_len < 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || num_blocks <= 0
        || max_blocks <= 0)
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size))
        return PKV_EUNSUPPORTED;
    if (B > 65535 || (int64_t)max_query_len > kMaxTokens)
        return PKV_EUNSUPPORTED;
    if (B == 0 || max_query_len == 0)
        return PKV_OK;
    if (!k_rows || !v_rows || !query_start || !k_cache || !v_cache || !block_tables
        || !context_lens)
        return PKV_EINVAL;
    const uintptr_t cache_align = one_byte(kv_dtype) ? 8 : 16;
    if (!aligned(k_rows, 16) || !aligned(v_rows, 16) || !aligned(k_cache, cache_align)
        || !aligned(v_cache, cache_align))
        return PKV_EINVAL;
    if (one_byte(kv_dtype) && (!k_scale || !v_scale))
        return PKV_EINVAL;
    pkv::WriteArgs a;
    a.k_rows = k_rows;
    a.v_rows = v_rows;
    a.query_start = query_start;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks = max_blocks;
    a.B = B;
    a.max_query_len = max_query_len;
    a.Hkv = Hkv;
    a.D = D;
    a.block_size = block_size;
    const Fmt f = format_of(kv_dtype, Hkv);
    a.kv_dtype = f.kvf;
    a.sc_blk = f.sc_blk;
    a.sc_head = f.sc_head;
    return launched(pkv::launch_write(a, (hipStream_t)stream));
}

// Beyond this many (new row, query head) columns per kv head the decode-
// shaped multi-query path would stream each context more than four times;
// the prefill kernel streams it once per 256 columns.
constexpr int64_t kPrefillColumns = 128;

// 16-column MFMA tiles per wave of the multi-query kernel: two once a kv
// head has more than 16 (new row, query head) columns.
static int mq_tiles_per_wave(int32_t max_query_len, int32_t G)
{
    return (int64_t)max_query_len * G > 16 ? 2 : 1;
}

static int mq_groups(int32_t Hkv, int32_t D, int32_t block_size, int32_t kv_dtype, int nct)
{
    return resident_groups(Hkv, D, block_size, kv_dtype, nct);
}

static int64_t mq_bytes(int ngroups, int32_t Hkv, int nct, int32_t D, int kvf)
{
    return schedule_bytes(ngroups, (int64_t)pkv::balanced_head_group(Hkv, nct, kvf) * 16 * nct, D);
}

int64_t paged_multiquery_workspace_size(int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                                        int32_t kv_dtype, int32_t max_query_len)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_query_len < 0)
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size) || Hq / Hkv > kMaxGroup
        || (int64_t)max_query_len > kMaxTokens)
        return PKV_EUNSUPPORTED;
    const int nct = mq_tiles_per_wave(max_query_len, Hq / Hkv);
    const int n = mq_groups(Hkv, D, block_size, kv_dtype, nct);
    if (n <= 0)
        return PKV_ELAUNCH;
    return mq_bytes(n, Hkv, nct, D, format_of(kv_dtype, Hkv).kvf);
}

int paged_multiquery_attention(const uint16_t* query, const int32_t* query_start,
                               int32_t total_rows, int32_t max_query_len, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int32_t max_blocks,
                               const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t block_size, int32_t num_blocks,
                               int32_t kv_dtype, float scale, void* workspace,
                               int64_t workspace_bytes, float* out, float* lse_out,
                               void* stream)
{
    if (B < 0 || total_rows < 0 || max_query_len < 0 || Hq <= 0 || Hkv <= 0 || D <= 0
        || block_size <= 0 || num_blocks <= 0 || max_blocks <= 0 || workspace_bytes < 0)
        return PKV_EINVAL;
    if (Hq % Hkv != 0 || !isfinite(scale))
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    if (!supported_d(D) || !supported_bs(block_size) || Hq / Hkv > kMaxGroup)
        return PKV_EUNSUPPORTED;
    if ((int64_t)max_blocks * block_size > kMaxTokens || (int64_t)max_query_len > kMaxTokens)
        return PKV_EUNSUPPORTED;
    if (B == 0 || total_rows == 0)
        return PKV_OK;
    if (max_query_len == 0)
        return PKV_EINVAL;                       // rows to attend but no new tokens
    if (!query || !query_start || !k_cache || !v_cache || !block_tables || !context_lens || !out
        || !workspace)
        return PKV_EINVAL;
    if (!aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)
        || !aligned(out, 16) || !aligned(workspace, 16) || (lse_out && !aligned(lse_out, 4)))
        return PKV_EINVAL;
    if (one_byte(kv_dtype) && (!k_scale || !v_scale))
        return PKV_EINVAL;
    const int32_t G = Hq / Hkv;
    const int nct = mq_tiles_per_wave(max_query_len, G);
    const int n = mq_groups(Hkv, D, block_size, kv_dtype, nct);
    if (n <= 0)
        return PKV_ELAUNCH;
    if (workspace_bytes < mq_bytes(n, Hkv, nct, D, format_of(kv_dtype, Hkv).kvf))
        return PKV_EINVAL;
    pkv::DecodeArgs a;
    a.query = query;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.lse_out = lse_out;
    a.partial_out = nullptr;
    a.partial_lse = nullptr;
    a.query_start = query_start;
    a.total_rows = total_rows;
    a.max_blocks = max_blocks;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.split_tokens = 0;
    a.max_splits = 1;
    a.scale_log2 = scale * 1.4426950408889634f;
    const Fmt fmt = format_of(kv_dtype, Hkv);
    a.sc_blk = fmt.sc_blk;
    a.sc_head = fmt.sc_head;
    pkv::BalanceArgs ws;
    ws.head_group = pkv::balanced_head_group(Hkv, nct, fmt.kvf);
    // as for a decode step: the Hkv / 4 four-head groups of a token range
    // run side by side
    ws.head_split = pkv::balanced_one_group_per_cu(Hkv, nct, fmt.kvf) ? Hkv / ws.head_group : 1;
    ws.ngroups_launched = n / ws.head_split * ws.head_split;
    carve_workspace(ws, workspace, (int64_t)ws.head_group * 16 * nct, D);
    // range boundaries in double precision: (tiles of the call) * (groups
    // launched) must stay below 2^52
    const int64_t ngroups = Hkv / ws.head_group;
    const int64_t col_groups = ((int64_t)max_query_len * G + 16 * nct - 1) / (16 * nct);
    const int64_t max_tiles =
        (int64_t)B * (((int64_t)max_blocks * block_size + 31) / 32) * col_groups * ngroups;
    if (max_tiles * ((int64_t)n + 1) >= ((int64_t)1 << 52))
        return PKV_EUNSUPPORTED;
    const bool nt = stream_kv_loads(num_blocks, block_size, Hkv, D, kv_dtype);
    if ((int64_t)max_query_len * G > kPrefillColumns)
        return launched(pkv::launch_prefill(a, max_query_len, D, block_size, fmt.kvf, nt,
                                            (hipStream_t)stream));
    return launched(pkv::launch_multiquery(a, ws, D, block_size, fmt.kvf, nct, nt,
                                           (hipStream_t)stream));
}

// Common checks of the block moves; fills block_bytes and scale_count.
static int move_checks(int32_t n, int32_t block_size, int32_t Hkv, int32_t D, int32_t num_blocks,
                       int32_t kv_dtype, pkv::BlockMoveArgs& a)
{
    if (n < 0 || block_size <= 0 || Hkv <= 0 || D <= 0 || num_blocks <= 0)
        return PKV_EINVAL;
    if (!valid_dtype(kv_dtype))
        return PKV_EINVAL;
    const int64_t esize = one_byte(kv_dtype) ? 1 : 2;
    a.block_bytes = (int64_t)block_size * Hkv * D * esize;
    if (a.block_bytes % 16 != 0)
        return PKV_EUNSUPPORTED;
    a.n = n;
    a.scale_count = scales_per_block(kv_dtype, Hkv);
    return PKV_OK;
}

static bool moves_aligned(const void* a, const void* b, const void* c, const void* d)
{
    return aligned(a, 16) && aligned(b, 16) && aligned(c, 16) && aligned(d, 16);
}

int paged_kv_gather_blocks(const void* k_cache, const void* v_cache, const float* k_scale,
                           const float* v_scale, const int32_t* block_ids, int32_t n,
                           int32_t block_size, int32_t Hkv, int32_t D, int32_t num_blocks,
                           int32_t kv_dtype, void* k_out, void* v_out, float* k_scale_out,
                           float* v_scale_out, void* stream)
{
    pkv::BlockMoveArgs a = {};
    int st = move_checks(n, block_size, Hkv, D, num_blocks, kv_dtype, a);
    if (st != PKV_OK || n == 0)
        return st;
    if (!k_cache || !v_cache || !block_ids || !k_out || !v_out)
        return PKV_EINVAL;
    if (!moves_aligned(k_cache, v_cache, k_out, v_out))
        return PKV_EINVAL;
    if (a.scale_count > 0 && (!k_scale || !v_scale || !k_scale_out || !v_scale_out))
        return PKV_EINVAL;
    a.src_k = (const unsigned char*)k_cache;
    a.src_v = (const unsigned char*)v_cache;
    a.dst_k = (unsigned char*)k_out;
    a.dst_v = (unsigned char*)v_out;
    a.src_ks = k_scale;
    a.src_vs = v_scale;
    a.dst_ks = k_scale_out;
    a.dst_vs = v_scale_out;
    a.src_ids = block_ids;
    a.dst_ids = nullptr;
    return launched(pkv::launch_move_blocks(a, (hipStream_t)stream));
}

int paged_kv_scatter_blocks(const void* k_in, const void* v_in, const float* k_scale_in,
                            const float* v_scale_in, const int32_t* block_ids, int32_t n,
                            int32_t block_size, int32_t Hkv, int32_t D, int32_t num_blocks,
                            int32_t kv_dtype, void* k_cache, void* v_cache, float* k_scale,
                            float* v_scale, void* stream)
{
    pkv::BlockMoveArgs a = {};
    int st = move_checks(n, block_size, Hkv, D, num_blocks, kv_dtype, a);
    if (st != PKV_OK || n == 0)
        return st;
    if (!k_in || !v_in || !block_ids || !k_cache || !v_cache)
        return PKV_EINVAL;
    if (!moves_aligned(k_in, v_in, k_cache, v_cache))
        return PKV_EINVAL;
    if (a.scale_count > 0 && (!k_scale || !v_scale || !k_scale_in || !v_scale_in))
        return PKV_EINVAL;
    a.src_k = (const unsigned char*)k_in;
    a.src_v = (const unsigned char*)v_in;
    a.dst_k = (unsigned char*)k_cache;
    a.dst_v = (unsigned char*)v_cache;
    a.src_ks = k_scale_in;
    a.src_vs = v_scale_in;
    a.dst_ks = k_scale;
    a.dst_vs = v_scale;
    a.src_ids = nullptr;
    a.dst_ids = block_ids;
    return launched(pkv::launch_move_blocks(a, (hipStream_t)stream));
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                         const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                         int32_t block_size, int32_t Hkv, int32_t D, int32_t num_blocks,
                         int32_t kv_dtype, void* stream)
{
    pkv::BlockMoveArgs a = {};
    int st = move_checks(n, block_size, Hkv, D, num_blocks, kv_dtype, a);
    if (st != PKV_OK || n == 0)
        return st;
    if (!k_cache || !v_cache || !src_ids || !dst_ids)
        return PKV_EINVAL;
    if (!moves_aligned(k_cache, v_cache, k_cache, v_cache))
        return PKV_EINVAL;
    if (a.scale_count > 0 && (!k_scale || !v_scale))
        return PKV_EINVAL;
    a.src_k = (const unsigned char*)k_cache;
    a.src_v = (const unsigned char*)v_cache;
    a.dst_k = (unsigned char*)k_cache;
    a.dst_v = (unsigned char*)v_cache;
    a.src_ks = k_scale;
    a.src_vs = v_scale;
    a.dst_ks = k_scale;
    a.dst_vs = v_scale;
    a.src_ids = src_ids;
    a.dst_ids = dst_ids;
    return launched(pkv::launch_move_blocks(a, (hipStream_t)stream));
}

int split_context_reduce(const float* partial_out, const float* partial_lse,
                         const int32_t* context_lens, int32_t B, int32_t Hq, int32_t D,
                         int32_t split_tokens, int32_t max_splits, float* out, float* lse_out,
                         void* stream)
{
    if (B < 0 || Hq <= 0 || D <= 0 || split_tokens <= 0 || max_splits <= 0)
        return PKV_EINVAL;
    if (D % 4 != 0 || D > 1024)
        return PKV_EUNSUPPORTED;
    if (B == 0)
        return PKV_OK;
    if (!partial_out || !partial_lse || !context_lens || !out)
        return PKV_EINVAL;
    if (!aligned(partial_out, 16) || !aligned(out, 16))
        return PKV_EINVAL;
    pkv::ReduceArgs a;
    a.partial_out = partial_out;
    a.partial_lse = partial_lse;
    a.context_lens = context_lens;
    a.out = out;
    a.lse_out = lse_out;
    a.B = B;
    a.Hq = Hq;
    a.D = D;
    a.split_tokens = split_tokens;
    a.max_splits = max_splits;
    return launched(pkv::launch_reduce(a, (hipStream_t)stream));
}

int pkv_stream_read(const void* buf, int64_t bytes, int32_t waves, uint32_t* sink,
                    void* stream)
{
    if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4))
        return PKV_EINVAL;
    if (waves <= 0 || waves % 4 != 0 || bytes <= 0 || bytes % ((int64_t)waves * 8192) != 0)
        return PKV_EINVAL;
    return launched(pkv::launch_stream_read(buf, bytes, waves, sink, (hipStream_t)stream));
}

} // extern "C"
