// prefill.hip -- causal attention of long runs of new tokens (prefill
// chunks) over a paged cache, for gfx950.
//
// Pages cited:
//   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
//        Attention Variants, and the Bandwidth Wall" -- "Continuous
//        Batching" (chunked prefill), "PagedAttention", "Attention
//        Variants" (GQA), "FP8 KV cache", "INT8 KV cache"
//
// Same operation as the multi-query path of decode.hip: row
// query_start[b] + i of sequence b is position p = T_b - q_b + i and
// attends over tokens [0, p] of kv head hq / G.  When a sequence brings
// many new tokens, the (row, head) pairs of one kv head are many MFMA
// columns, and giving every 32 of them their own pass over the context (as
// the decode-shaped path does) would read the context once per 32 columns.
// Here a work-group of 8 waves takes 256 columns of one (sequence, kv head)
// and streams the context once for all of them: each 64-token tile of K and
// V is loaded by the whole group, converted to bf16 and staged in LDS as
// rows (double-buffered, one barrier per tile); every wave then forms its
// two 16-column score tiles from LDS K, runs the online softmax and
// accumulates V^T . P^T, its V^T operands fetched with the transposing
// LDS read, as the decode tile body does.  (64-token tiles halve the
// barriers and per-tile fixed work of 32-token ones: +4% bf16, +7-8% for
// the 1-byte formats.)
// Work-groups that share a (sequence, kv head) are placed on one XCD so
// their re-reads of the context hit that XCD's L2.
//
// fp8 codes become exact bf16 values in LDS and the block scales enter
// through the scores (K) and probabilities (V); int8 codes become the
// exact bf16 integers u - zp.
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kPWaves = 8;                         // waves per work-group
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPCols = 32;                         // MFMA columns per wave
constexpr int kPGroupCols = kPWaves * kPCols;      // columns per work-group
constexpr int kPTile = 64;                         // tokens per staged tile
constexpr int kPHalves = kPTile / 16;              // 16-token MFMA row tiles per tile
constexpr int kPGroups = kPTile / 32;              // 32-token PV contraction groups
constexpr int kXcds = 8;
// Largest lag (log2 units) of a column's reference max behind its running
// max: probabilities stay <= 2^8.
constexpr float kMaxLag = 8.f;

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

template <int D, int KVF>
struct PCfg {
    static constexpr int ESZ = KVF ? 1 : 2;
    static constexpr int ROW_BYTES = D * ESZ;          // one cached token row
    static constexpr int CPR = ROW_BYTES / 16;         // 16-byte chunks per row
    static constexpr int NCHUNK = kPTile * CPR;        // chunks per K (or V) tile
    static constexpr int CPT = (2 * NCHUNK + kPThreads - 1) / kPThreads;  // per thread
    static constexpr int KPITCH = D * 2 + 16;          // bf16 K row pitch in LDS
    // bf16 V row pitch: eight consecutive rows on disjoint banks for the
    // transposing reads
    static constexpr int VPITCH = D * 2 + 32;
    static constexpr int KBYTES = kPTile * KPITCH;
    // 1-byte formats: the K and V scales of the tile's 16-token quarters
    static constexpr int SCALES = KBYTES + kPTile * VPITCH;
    static constexpr int BUF = SCALES + 8 * kPHalves;
    static constexpr int KSTEPS = D / 32;
    static constexpr int DT = D / 16;
};

template <int NT>
__device__ __forceinline__ u32x4 pload(const unsigned char* p)
{
    if (NT)
        return __builtin_nontemporal_load((const u32x4*)p);
    return *(const u32x4*)p;
}


template <int D, int BS, int KVF, int NT>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(DecodeArgs a, int32_t units,
                                                            int32_t row_blocks)
{
    using C = PCfg<D, KVF>;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];   // 2 tile buffers

    // XCD-aware unit order: consecutive units (the row blocks of one
    // sequence and kv head) run on one XCD.
    const int per_xcd = (units + kXcds - 1) / kXcds;
    const int unit = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (unit >= units || blockIdx.x / kXcds >= per_xcd)
        return;
    const int rb = unit % row_blocks;
    const int bh = unit / row_blocks;
    const int h = bh % a.Hkv;
    const int b = bh / a.Hkv;
    const int qs = a.query_start[b];
    const int q = a.query_start[b + 1] - qs;
    const int G = a.G;
    if (rb * kPGroupCols >= q * G)
        return;                                           // uniform over the group
    const int T = a.context_lens[b];
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int q4 = lane >> 4;
    const int r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // this group's last row and its causal limit bound the token range
    const int last_col = min(q * G, (rb + 1) * kPGroupCols) - 1;
    const int t_end = T - q + last_col / G + 1;

    // this lane's two columns
    int lim[2], qrow[2], hq[2];
    bool live[2];
    bf16x8 qf[2][C::KSTEPS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = rb * kPGroupCols + wave * kPCols + 16 * j + r16;
        const int i = c / G;
        live[j] = i < q;
        qrow[j] = qs + (live[j] ? i : 0);
        hq[j] = h * G + (c - i * G);
        lim[j] = live[j] ? T - q + i + 1 : 0;
        const uint16_t* qp = a.query + ((size_t)qrow[j] * a.Hq + (live[j] ? hq[j] : 0)) * D;
#pragma unroll
        for (int k = 0; k < C::KSTEPS; ++k) {
            u32x4 v = *(const u32x4*)(qp + 8 * (q4 + 4 * k));
            if (!live[j])
                v = u32x4{0u, 0u, 0u, 0u};
            qf[j][k] = as_bf16x8(v);
        }
    }
    // wave-uniform bounds of the wave's columns
    const int wc0 = rb * kPGroupCols + wave * kPCols;
    const int w_first = min(wc0, q * G - 1) / G;
    const int w_last = min(wc0 + kPCols, q * G) - 1;
    const int wave_from = T - q + w_first + 1;           // no column's limit below
    const int wave_end = wc0 < q * G ? T - q + w_last / G + 1 : 0;

    const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
    const unsigned char* kc = (const unsigned char*)a.k_cache;
    const unsigned char* vc = (const unsigned char*)a.v_cache;
    const size_t tok_stride = (size_t)a.Hkv * C::ROW_BYTES;
    const size_t head_off = (size_t)h * C::ROW_BYTES;

    auto scale_at = [&](const float* s, int p, int off) -> float {
        return s[(size_t)p * a.sc_blk + (size_t)h * a.sc_head + off];
    };

    // Cooperative load of one tile's chunks into registers.  Thread chunk u
    // is the same (row, 16-byte column) of K or V in every tile; its block-
    // table entry is read one tile ahead, so a tile's loads never wait on a
    // table read.
    int ch_row[C::CPT];
    bool ch_ok[C::CPT], ch_v[C::CPT];
    uint32_t ch_off[C::CPT];
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
        const int c = tid + u * kPThreads;
        ch_ok[u] = c < 2 * C::NCHUNK;
        const int kv = c / C::NCHUNK;
        const int rem = c - kv * C::NCHUNK;
        ch_v[u] = kv != 0;
        ch_row[u] = rem / C::CPR;
        ch_off[u] = (uint32_t)((ch_row[u] % BS) * tok_stride + head_off)
                    + 16u * (uint32_t)(rem - ch_row[u] * C::CPR);
    }
    int pblk[C::CPT];              // physical block of each chunk of the next tile (-1: none)
    auto load_tbl = [&](int t0) {
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            const int t = t0 + ch_row[u];
            pblk[u] = (ch_ok[u] && t < t_end) ? trow[t / BS] : -1;
        }
    };
    // 1-byte formats: the chunk's zero point (int8), and for the first chunk
    // of each 16-token row group the K or V scale of those rows, loaded with
    // the chunk and handed to every wave through LDS by stage()
    bool ch_scale_slot[C::CPT];
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
        const int c = tid + u * kPThreads;
        ch_scale_slot[u] = ch_ok[u] && (ch_row[u] & 15) == 0
                           && (c - (ch_v[u] ? C::NCHUNK : 0)) % C::CPR == 0;
    }
    u32x4 reg[C::CPT];
    float zp_cur[C::CPT], sc_cur[C::CPT];
    auto fetch = [&](int t0) {
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            reg[u] = u32x4{0u, 0u, 0u, 0u};
            zp_cur[u] = 0.f;
            if (pblk[u] >= 0) {
                reg[u] = pload<NT>((ch_v[u] ? vc : kc) + (size_t)pblk[u] * BS * tok_stride
                                   + ch_off[u]);
                if (KVF == 2)
                    zp_cur[u] = scale_at(ch_v[u] ? a.v_scale : a.k_scale, pblk[u], 1);
            }
        }
#pragma unroll
        for (int u = 0; u < C::CPT; ++u)
            if (KVF && ch_scale_slot[u])
                sc_cur[u] = pblk[u] >= 0 ? scale_at(ch_v[u] ? a.v_scale : a.k_scale, pblk[u], 0)
                                         : 1.f;
        load_tbl(t0 + kPTile);
    };
    // registers -> bf16 rows of LDS buffer `buf`
    auto stage = [&](int t0, int buf) {
        unsigned char* kl = lds + buf * C::BUF;
        unsigned char* vl = kl + C::KBYTES;
#pragma unroll
        for (int u = 0; u < C::CPT; ++u) {
            const int c = tid + u * kPThreads;
            if (c >= 2 * C::NCHUNK)
                continue;
            const int kv = c / C::NCHUNK;
            const int rem = c - kv * C::NCHUNK;
            const int row = rem / C::CPR;
            const int col = rem - row * C::CPR;
            unsigned char* dst = kv ? vl + row * C::VPITCH : kl + row * C::KPITCH;
            if (!KVF) {
                u32x2* d2 = (u32x2*)(dst + 16 * col);
                d2[0] = u32x2{reg[u][0], reg[u][1]};
                d2[1] = u32x2{reg[u][2], reg[u][3]};
            } else {
                u32x4 lo, hi;
                const int t = t0 + row;
                if (KVF == 1) {
                    fp8x16_to_bf16x16(reg[u], lo, hi);
                } else {
                    u8x16_to_bf16x16(reg[u], zp_cur[u], lo, hi);
                    if (t >= t_end) {
                        lo = u32x4{0u, 0u, 0u, 0u};
                        hi = u32x4{0u, 0u, 0u, 0u};
                    }
                }
                u32x2* d2 = (u32x2*)(dst + 32 * col);
                d2[0] = u32x2{lo[0], lo[1]};
                d2[1] = u32x2{lo[2], lo[3]};
                d2[2] = u32x2{hi[0], hi[1]};
                d2[3] = u32x2{hi[2], hi[3]};
            }
        }
        // [K quarter 0 .. kPHalves - 1, V quarter 0 .. kPHalves - 1]
#pragma unroll
        for (int u = 0; u < C::CPT; ++u)
            if (KVF && ch_scale_slot[u])
                ((float*)(kl + C::SCALES))[kPHalves * (int)ch_v[u] + ch_row[u] / 16] = sc_cur[u];
    };

    f32x4 acc[2][C::DT];
    float m_run[2], l_run[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            acc[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[j] = -__builtin_inff();
        l_run[j] = 0.f;
    }
    const float sl2 = a.scale_log2;
    const uint32_t tr_off0 = (uint32_t)(4 * q4 + (r16 >> 2)) * C::VPITCH + 8 * (r16 & 3);

    // masked: some column's causal limit falls inside the tile (a
    // compile-time flag, so unmasked tiles carry no per-score selects)
    auto compute = [&](int t0, int buf, auto masked_c) {
        constexpr bool masked = decltype(masked_c)::value;
        const unsigned char* kl = lds + buf * C::BUF;
        const unsigned char* vl = kl + C::KBYTES;
        float ks[kPHalves], vs[kPHalves];
#pragma unroll
        for (int tau = 0; tau < kPHalves; ++tau) {
            ks[tau] = 1.f;
            vs[tau] = 1.f;
        }
        if (KVF) {
            const float* sc = (const float*)(kl + C::SCALES);
#pragma unroll
            for (int tau = 0; tau < kPHalves; ++tau) {
                ks[tau] = sc[tau];
                vs[tau] = sc[kPHalves + tau];
            }
        }
        // Wave priority is raised over the matrix-core sections: of the two
        // waves sharing a SIMD, the one holding matrix work issues it first
        // and the other's softmax fills the VALU meanwhile (measured +5%).
        f32x4 sacc[2][kPHalves];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int tau = 0; tau < kPHalves; ++tau) {
            sacc[0][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
            sacc[1][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < C::KSTEPS; ++k) {
                const u32x4 kw =
                    *(const u32x4*)(kl + (16 * tau + r16) * C::KPITCH + 16 * (q4 + 4 * k));
                sacc[0][tau] = mfma_16x16x32(as_bf16x8(kw), qf[0][k], sacc[0][tau]);
                sacc[1][tau] = mfma_16x16x32(as_bf16x8(kw), qf[1][k], sacc[1][tau]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // P operands per 32-token group g: contraction slot (q4, i) holds
        // token 32 g + 4 q4 + i (i < 4) or 32 g + 16 + 4 q4 + i - 4
        bf16x8 pb[kPGroups][2], pb_lo[kPGroups][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // scores relative to the column's reference max (0 while nothing
            // is visible), which may trail the running max by up to kMaxLag
            const float m_ref = m_run[j] == -__builtin_inff() ? 0.f : m_run[j];
            float s[4 * kPHalves];
#pragma unroll
            for (int tau = 0; tau < kPHalves; ++tau) {
                const float f = KVF ? sl2 * ks[tau] : sl2;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = __builtin_fmaf(sacc[j][tau][i], f, -m_ref);
                    if (masked && t0 + 16 * tau + 4 * q4 + i >= lim[j])
                        x = -__builtin_inff();
                    s[4 * tau + i] = x;
                }
            }
            float lm = s[0];
#pragma unroll
            for (int i = 1; i < 4 * kPHalves; ++i)
                lm = fmaxf(lm, s[i]);
            // rescale only on a column's first visible tile or when a tile
            // raises its max by more than kMaxLag (decided for the wave)
            if (__builtin_amdgcn_ballot_w64(lm > kMaxLag || m_run[j] == -__builtin_inff())) {
                float mt = lm;
                mt = fmaxf(mt, xor_shuffle(mt, 16));
                mt = fmaxf(mt, xor_shuffle(mt, 32));
                const float m_new = fmaxf(m_run[j], m_ref + mt);
                const float m_ref_new = m_new == -__builtin_inff() ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_ref_new);
                const float delta = m_ref_new - m_ref;
#pragma unroll
                for (int i = 0; i < 4 * kPHalves; ++i)
                    s[i] -= delta;
                m_run[j] = m_new;
                l_run[j] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
                    acc[j][dt] *= alpha;
            }
            float p[4 * kPHalves];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4 * kPHalves; ++i) {
                p[i] = __builtin_amdgcn_exp2f(s[i]);
                psum += p[i];
            }
            l_run[j] += psum;
            if (KVF) {
#pragma unroll
                for (int i = 0; i < 4 * kPHalves; ++i)
                    p[i] *= vs[i / 4];
            }
            // P as hi + lo bf16 terms (about 16 significant bits)
#pragma unroll
            for (int g = 0; g < kPGroups; ++g) {
                u32x4 pw, pr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = p[8 * g + 2 * i], p1 = p[8 * g + 2 * i + 1];
                    pw[i] = pack_bf16x2(p0, p1);
                    pr[i] = pack_bf16x2(p0 - bf16_bits_to_f32(pw[i] & 0xFFFFu),
                                        p1 - bf16_bits_to_f32(pw[i] >> 16));
                }
                pb[g][j] = as_bf16x8(pw);
                pb_lo[g][j] = as_bf16x8(pr);
            }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
            for (int g = 0; g < kPGroups; ++g) {
            // contraction slots of group g: lane (q4, 4e + k) names token
            // 32 g + 4q4 + e (then 32 g + 16 + 4q4 + e) at head-dim 16 dt + 4k,
            // and receives column 16 dt + r16 of the four
            const unsigned char* vg = vl + 32 * g * C::VPITCH + tr_off0 + 32 * dt;
            const u32x2 a0 = lds_read_tr16(vg);
            const u32x2 a1 = lds_read_tr16(vg + 16 * C::VPITCH);
            const u32x4 vw = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[j][dt] = mfma_16x16x32(as_bf16x8(vw), pb[g][j], acc[j][dt]);
                acc[j][dt] = mfma_16x16x32(as_bf16x8(vw), pb_lo[g][j], acc[j][dt]);
            }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // pipeline: the next tile's loads are in flight while this one is
    // computed; one barrier per tile hands the buffers over
    const int ntiles = (t_end + kPTile - 1) / kPTile;
    // tiles below every causal limit of the group (wave 0 holds its lowest
    // rows): no masking; the loop bounds are uniform over the group, so
    // every wave meets every barrier
    const int group_from = T - q + (rb * kPGroupCols) / G + 1;
    const int n_plain = min(ntiles, group_from / kPTile);
    auto iteration = [&](int it, auto masked_c) {
        const int t0 = it * kPTile;
        const bool more = it + 1 < ntiles;
        if (more)
            fetch(t0 + kPTile);
        if (t0 < wave_end)
            compute(t0, it & 1, masked_c);
        if (more)
            stage(t0 + kPTile, (it + 1) & 1);
        __syncthreads();
    };
    load_tbl(0);
    fetch(0);
    stage(0, 0);
    __syncthreads();
    for (int it = 0; it < n_plain; ++it)
        iteration(it, Flag<false>());
    for (int it = n_plain; it < ntiles; ++it)
        iteration(it, Flag<true>());

#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float l = l_run[j];
        l += xor_shuffle(l, 16);
        l += xor_shuffle(l, 32);
        if (!live[j])
            continue;
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        const size_t orow = (size_t)qrow[j] * a.Hq + hq[j];
        float* o = a.out + orow * D;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            *(f32x4*)(o + 16 * dt + 4 * q4) = acc[j][dt] * inv;
        if (a.lse_out && q4 == 0)
            a.lse_out[orow] = (m_run[j] + __builtin_log2f(l)) * kLn2;
    }
}

template <int D, int BS, int KVF>
hipError_t launch_prefill_t(const DecodeArgs& a, int max_query_len, bool nt, hipStream_t stream)
{
    const long long row_blocks =
        ((long long)max_query_len * a.G + kPGroupCols - 1) / kPGroupCols;
    const long long units = (long long)a.B * a.Hkv * row_blocks;
    if (units <= 0)
        return hipSuccess;
    const long long groups = (units + kXcds - 1) / kXcds * kXcds;
    if (groups > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    const size_t lds = 2 * (size_t)PCfg<D, KVF>::BUF;
    // two tile buffers exceed 64 KB at D = 128: allow the kernel that much
    // dynamic LDS (gfx950 has 160 KB per CU); set on every call, so it holds
    // for whichever device is current (a host-side call, no GPU work)
    const void* fn = nt ? reinterpret_cast<const void*>(&prefill_kernel<D, BS, KVF, 1>)
                        : reinterpret_cast<const void*>(&prefill_kernel<D, BS, KVF, 0>);
    const hipError_t attr =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess)
        return attr;
    if (nt)
        hipLaunchKernelGGL((prefill_kernel<D, BS, KVF, 1>), dim3((unsigned)groups),
                           dim3(kPThreads), lds, stream, a, (int32_t)units, (int32_t)row_blocks);
    else
        hipLaunchKernelGGL((prefill_kernel<D, BS, KVF, 0>), dim3((unsigned)groups),
                           dim3(kPThreads), lds, stream, a, (int32_t)units, (int32_t)row_blocks);
    return hipGetLastError();
}

} // namespace

hipError_t launch_prefill(const DecodeArgs& a, int max_query_len, int D, int block_size,
                          int kvf, bool nt, hipStream_t stream)
{
#define PKV_PF(d, bs)                                                                   \
    if (D == d && block_size == bs)                                                    \
        return kvf == 2   ? launch_prefill_t<d, bs, 2>(a, max_query_len, nt, stream)    \
               : kvf == 1 ? launch_prefill_t<d, bs, 1>(a, max_query_len, nt, stream)    \
                          : launch_prefill_t<d, bs, 0>(a, max_query_len, nt, stream);
    PKV_PF(128, 16)
    PKV_PF(128, 32)
    PKV_PF(64, 16)
    PKV_PF(64, 32)
#undef PKV_PF
    return hipErrorInvalidValue;
}

} // namespace pkv
