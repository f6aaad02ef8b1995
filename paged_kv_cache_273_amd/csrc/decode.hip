// decode.hip -- paged decode attention for gfx950 (MI355X).
//
// Pages cited:
//   [A] "KV-Cache Engineering: Paged Attention, Prefix Cache,
//        Disaggregation (2026)"
//   [B] "KV Cache Engineering: PagedAttention, Continuous Batching,
//        Attention Variants, and the Bandwidth Wall"
//
// What it computes: for each sequence b and query head hq, softmax
// attention of query[b, hq] over the T_b cached tokens of kv head
// hq / G, each token found through the block table ([B] "PagedAttention";
// GQA grouping from [B] "Attention Variants").  Decode reads every cached
// byte once per generated token, so the kernel is an HBM stream ([B] "Two
// Costs: Capacity and Bandwidth").
//
// Work unit: one wave = (sequence b, kv head h, token range).  The range
// is the whole context (single pass) or one split of `split_tokens`.
// Units of the same (b, split) for consecutive kv heads are neighbouring
// waves of one work-group, so the group streams whole physical blocks
// ([num_blocks, bs, Hkv, D] keeps the Hkv rows of a slot contiguous).
//
// Per 32-token tile a wave:
//   * loads K straight into the matrix-core operand layout: lane (q, r)
//     holds 16 bytes of token r's row;
//   * loads V coalesced (whole 256-byte rows per 16 lanes) and stages it
//     in its own LDS slice, converting fp8 codes to bf16 on the way;
//   * S^T[token][head] = K . Q^T on the 16x16x32 bf16 MFMA: the G query
//     heads of the group (padded to 16 columns) share every K load;
//   * online softmax over the tile in fp32 (exp2 domain), the max taken
//     across the wave with two lane butterflies;
//   * O^T[d][head] += V^T . P^T on the MFMA, V^T read from LDS with a
//     transposing 16-bit gather (row pitch padded by 8 bytes so the four
//     lane groups hit disjoint banks); P enters as a hi + lo pair of bf16
//     terms so the probabilities keep ~16 significant bits.
// The next tile's K/V loads are issued before the current tile is
// processed, so every wave keeps ~16 KB in flight.
//
// The last tile of a range is masked: tokens at or past the range end
// have their score selected to -inf and their V row zeroed before it
// reaches LDS (the cache may hold NaN there: selection, not
// multiplication, keeps it out).  Block-table entries past the last live
// block are never dereferenced.
//
// FP8 ([B] "FP8 KV cache"): E4M3FN codes convert exactly to bf16; the
// per-(block, kv head) scale multiplies the block's scores (K) and the
// block's probabilities before the PV product (V).
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kTile = 32;

template <int D, int FP8>
struct Cfg {
    static constexpr int ESZ = FP8 ? 1 : 2;            // bytes per cached element
    static constexpr int ROW_BYTES = D * ESZ;           // one token of one kv head
    static constexpr int KSTEPS = D / 32;               // MFMA k-steps of q . k
    static constexpr int K_LOADS = FP8 ? D / 64 : D / 32;  // 16-B loads per lane per 16 tokens
    static constexpr int V_LPR = ROW_BYTES / 16;        // lanes per V row
    static constexpr int V_RPI = kWave / V_LPR;         // V rows per load instruction
    static constexpr int V_LOADS = kTile / V_RPI;       // V loads per tile
    static constexpr int DT = D / 16;                   // 16-wide d tiles of the output
    static constexpr int PITCH = D * 2 + 8;             // LDS row pitch (bf16 rows), bytes
    static constexpr int LDS_BYTES = kTile * PITCH;     // per wave
    static_assert(16 % V_RPI == 0, "a V load must stay inside one 16-token block");
};

// First of the 8 consecutive head-dim elements that lane group q feeds to
// MFMA k-step j.  bf16: one 16-byte load per k-step (chunk q + 4j of
// 8 elements).  fp8: one 16-byte load holds two k-steps (chunk q + 4c of
// 16 codes, c = j / 2, low or high half).
template <int FP8>
__device__ __forceinline__ int kdim_base(int j, int q)
{
    return FP8 ? 16 * (q + 4 * (j >> 1)) + 8 * (j & 1) : 8 * (q + 4 * j);
}

// Token (within the 32-token tile) held in contraction slot (q, i) of the
// PV product: the S^T output of tile 0 gives lane group q tokens 4q..4q+3,
// tile 1 gives 16+4q..16+4q+3.
__device__ __forceinline__ int pv_token(int q, int i)
{
    return i < 4 ? 4 * q + i : 16 + 4 * q + (i - 4);
}

template <int D, int FP8>
struct Tile {
    u32x4 k[2][Cfg<D, FP8>::K_LOADS];
    u32x4 v[Cfg<D, FP8>::V_LOADS];
    int pA, pB;            // physical blocks of tokens 0..15 / 16..31
    float ksA, ksB, vsA, vsB;
};

template <int D, int BS, int FP8, bool SPLIT>
__global__ __launch_bounds__(kWavesPerGroup * kWave, 2)
void decode_kernel(DecodeArgs a)
{
    using C = Cfg<D, FP8>;
    __shared__ __attribute__((aligned(16))) unsigned char lds_all[kWavesPerGroup * C::LDS_BYTES];

    const int lane = __lane_id();
    const int q4 = lane >> 4;
    const int r16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = blockIdx.x * kWavesPerGroup + wave;

    const int Hkv = a.Hkv;
    const int h = unit % Hkv;
    int rest = unit / Hkv;
    int split = 0;
    if (SPLIT) {
        split = rest % a.max_splits;
        rest /= a.max_splits;
    }
    const int b = rest;
    if (b >= a.B)
        return;
    const int T = a.context_lens[b];
    int t_begin = 0, t_end = T;
    if (SPLIT) {
        t_begin = split * a.split_tokens;
        if (t_begin >= T)
            return;
        t_end = min(T, t_begin + a.split_tokens);
    }
    const int G = a.G;
    const int hq = h * G + r16;              // this lane's query head column
    const bool live_col = r16 < G;

    if (t_end <= t_begin) {                  // empty sequence, single pass
        if (live_col) {
            float* o = a.out + ((size_t)b * a.Hq + hq) * D;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                *(f32x4*)(o + 16 * dt + 4 * q4) = f32x4{0.f, 0.f, 0.f, 0.f};
            if (a.lse_out && q4 == 0)
                a.lse_out[(size_t)b * a.Hq + hq] = -__builtin_inff();
        }
        return;
    }

    // Q^T operand: column r16 = query head h*G + r16 (zero past G).
    bf16x8 qf[C::KSTEPS];
    {
        const uint16_t* qrow = a.query + ((size_t)b * a.Hq + (live_col ? hq : 0)) * D;
#pragma unroll
        for (int j = 0; j < C::KSTEPS; ++j) {
            u32x4 v = *(const u32x4*)(qrow + kdim_base<FP8>(j, q4));
            if (!live_col)
                v = u32x4{0u, 0u, 0u, 0u};
            qf[j] = as_bf16x8(v);
        }
    }

    // Block-table window of this unit, 64 entries per VGPR load.
    const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
    const int j_first = t_begin / BS;
    const int j_last = (t_end - 1) / BS;
    int tbl_base = -1;
    int tbl = 0;
    auto phys = [&](int j) -> int {
        int jj = min(j, j_last) - j_first;
        int base = jj & ~63;
        if (base != tbl_base) {
            tbl_base = base;
            int idx = j_first + base + lane;
            tbl = (idx <= j_last) ? trow[idx] : 0;
        }
        return __builtin_amdgcn_readlane(tbl, jj - base);
    };

    const unsigned char* kc = (const unsigned char*)a.k_cache;
    const unsigned char* vc = (const unsigned char*)a.v_cache;
    const size_t tok_stride = (size_t)Hkv * C::ROW_BYTES;
    const size_t head_off = (size_t)h * C::ROW_BYTES;

    auto load_tile = [&](int t0, Tile<D, FP8>& tl) {
        if (BS == 16) {
            tl.pA = phys(t0 / 16);
            tl.pB = phys(t0 / 16 + 1);
        } else {
            tl.pA = phys(t0 / 32);
            tl.pB = tl.pA;
        }
        if (FP8) {
            tl.ksA = a.k_scale[(size_t)tl.pA * Hkv + h];
            tl.vsA = a.v_scale[(size_t)tl.pA * Hkv + h];
            tl.ksB = a.k_scale[(size_t)tl.pB * Hkv + h];
            tl.vsB = a.v_scale[(size_t)tl.pB * Hkv + h];
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int p = tau ? tl.pB : tl.pA;
            const int slot = BS == 16 ? r16 : 16 * tau + r16;
            const unsigned char* src = kc + ((size_t)p * BS + slot) * tok_stride + head_off;
#pragma unroll
            for (int c = 0; c < C::K_LOADS; ++c)
                tl.k[tau][c] = *(const u32x4*)(src + 16 * (q4 + 4 * c));
        }
#pragma unroll
        for (int k = 0; k < C::V_LOADS; ++k) {
            const int r = k * C::V_RPI + lane / C::V_LPR;
            const int p = (BS == 16 && k * C::V_RPI >= 16) ? tl.pB : tl.pA;
            const int slot = BS == 16 ? (r & 15) : r;
            const unsigned char* src = vc + ((size_t)p * BS + slot) * tok_stride + head_off;
            tl.v[k] = *(const u32x4*)(src + 16 * (lane % C::V_LPR));
        }
    };

    unsigned char* lds = lds_all + wave * C::LDS_BYTES;
    f32x4 acc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
        acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();
    float l_run = 0.f;
    const float sl2 = a.scale_log2;

    auto compute_tile = [&](int t0, const Tile<D, FP8>& tl, bool masked) {
        // V rows -> LDS as bf16 (zeroed past the range end)
#pragma unroll
        for (int k = 0; k < C::V_LOADS; ++k) {
            const int r = k * C::V_RPI + lane / C::V_LPR;
            const int c = lane % C::V_LPR;
            u32x4 v = tl.v[k];
            if (masked && t0 + r >= t_end)
                v = u32x4{0u, 0u, 0u, 0u};
            if (FP8) {
                u32x4 lo, hi;
                fp8x16_to_bf16x16(v, lo, hi);
                u32x2* dst = (u32x2*)(lds + r * C::PITCH + 32 * c);
                dst[0] = u32x2{lo[0], lo[1]};
                dst[1] = u32x2{lo[2], lo[3]};
                dst[2] = u32x2{hi[0], hi[1]};
                dst[3] = u32x2{hi[2], hi[3]};
            } else {
                u32x2* dst = (u32x2*)(lds + r * C::PITCH + 16 * c);
                dst[0] = u32x2{v[0], v[1]};
                dst[1] = u32x2{v[2], v[3]};
            }
        }

        // scores S^T[token][head] for the two 16-token halves
        f32x4 sacc[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            sacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < C::K_LOADS; ++c) {
                if (FP8) {
                    u32x4 lo, hi;
                    fp8x16_to_bf16x16(tl.k[tau][c], lo, hi);
                    sacc[tau] = mfma_16x16x32(as_bf16x8(lo), qf[2 * c], sacc[tau]);
                    sacc[tau] = mfma_16x16x32(as_bf16x8(hi), qf[2 * c + 1], sacc[tau]);
                } else {
                    sacc[tau] = mfma_16x16x32(as_bf16x8(tl.k[tau][c]), qf[c], sacc[tau]);
                }
            }
        }

        float s[8];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const float f = FP8 ? sl2 * (tau ? tl.ksB : tl.ksA) : sl2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = sacc[tau][i] * f;
                if (masked && t0 + 16 * tau + 4 * q4 + i >= t_end)
                    x = -__builtin_inff();
                s[4 * tau + i] = x;
            }
        }
        float mt = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            mt = fmaxf(mt, s[i]);
        mt = fmaxf(mt, xor_shuffle(mt, 16));
        mt = fmaxf(mt, xor_shuffle(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
            psum += p[i];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            acc[dt] *= alpha;
        if (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] *= tl.vsA;
                p[4 + i] *= tl.vsB;
            }
        }
        // P as a two-term bf16 split, p = hi + lo (about 16 significant
        // bits): one bf16 term alone loses too much when V terms cancel.
        u32x4 pw, pr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pw[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
            pr[i] = pack_bf16x2(p[2 * i] - bf16_bits_to_f32(pw[i] & 0xFFFFu),
                                p[2 * i + 1] - bf16_bits_to_f32(pw[i] >> 16));
        }
        const bf16x8 pb = as_bf16x8(pw);
        const bf16x8 pb_lo = as_bf16x8(pr);

        // O^T[d][head] += V^T . P^T, V^T gathered from LDS
        const unsigned short* l16 = (const unsigned short*)lds;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            u32x4 vw;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                uint32_t lo = l16[(pv_token(q4, i) * C::PITCH) / 2 + 16 * dt + r16];
                uint32_t hi = l16[(pv_token(q4, i + 1) * C::PITCH) / 2 + 16 * dt + r16];
                vw[i / 2] = lo | (hi << 16);
            }
            acc[dt] = mfma_16x16x32(as_bf16x8(vw), pb, acc[dt]);
            acc[dt] = mfma_16x16x32(as_bf16x8(vw), pb_lo, acc[dt]);
        }
    };

    const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
    Tile<D, FP8> cur;
    load_tile(t_begin, cur);
    for (int it = 0; it < ntiles - 1; ++it) {
        Tile<D, FP8> nxt;
        load_tile(t_begin + kTile * (it + 1), nxt);
        compute_tile(t_begin + kTile * it, cur, false);
        cur = nxt;
    }
    compute_tile(t_begin + kTile * (ntiles - 1), cur, true);

    // normaliser: sum the four lane groups of each head column
    float l = l_run;
    l += xor_shuffle(l, 16);
    l += xor_shuffle(l, 32);
    const float inv = 1.0f / l;
    const float lse = (m_run + __builtin_log2f(l)) * kLn2;
    if (!live_col)
        return;
    float* o;
    if (SPLIT) {
        const size_t row = ((size_t)b * a.Hq + hq) * a.max_splits + split;
        o = a.partial_out + row * D;
        if (q4 == 0)
            a.partial_lse[row] = lse;
    } else {
        o = a.out + ((size_t)b * a.Hq + hq) * D;
        if (a.lse_out && q4 == 0)
            a.lse_out[(size_t)b * a.Hq + hq] = lse;
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
        *(f32x4*)(o + 16 * dt + 4 * q4) = acc[dt] * inv;
}

template <int D, int BS, int FP8>
hipError_t launch_d_bs_dt(const DecodeArgs& a, hipStream_t stream)
{
    const bool split = a.split_tokens > 0;
    const long long units = (long long)a.B * a.Hkv * (split ? a.max_splits : 1);
    const long long groups = (units + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups <= 0)
        return hipSuccess;
    if (groups > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)groups), block(kWavesPerGroup * kWave);
    if (split)
        hipLaunchKernelGGL((decode_kernel<D, BS, FP8, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<D, BS, FP8, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_d_bs(const DecodeArgs& a, int kv_dtype, hipStream_t stream)
{
    return kv_dtype == 1 ? launch_d_bs_dt<D, BS, 1>(a, stream)
                         : launch_d_bs_dt<D, BS, 0>(a, stream);
}

} // namespace

hipError_t launch_decode(const DecodeArgs& a, int D, int block_size, int kv_dtype,
                         hipStream_t stream)
{
    if (D == 128)
        return block_size == 16 ? launch_d_bs<128, 16>(a, kv_dtype, stream)
                                : launch_d_bs<128, 32>(a, kv_dtype, stream);
    return block_size == 16 ? launch_d_bs<64, 16>(a, kv_dtype, stream)
                            : launch_d_bs<64, 32>(a, kv_dtype, stream);
}

} // namespace pkv
