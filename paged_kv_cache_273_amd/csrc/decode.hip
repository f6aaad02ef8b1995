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
//     holds 16 bytes of token r's row (fp8 caches of 32-token blocks: K is
//     loaded like V, whole 128-byte rows, and staged in LDS, from where
//     each lane reads its operand bytes; 5% faster on such caches);
//   * loads V coalesced (whole 256-byte rows per 16 lanes) and stages it
//     in its own LDS slice, converting fp8 codes to bf16 on the way;
//   * S^T[token][head] = K . Q^T on the 16x16x32 bf16 MFMA: the G query
//     heads of the group (padded to 16 columns) share every K load;
//   * online softmax over the tile in fp32 (exp2 domain) against a
//     reference max that may trail the running max by up to 8 (so the
//     accumulators are rescaled only on the few tiles that raise it more);
//   * O^T[d][head] += V^T . P^T on the MFMA, V^T read from LDS with the
//     transposing 16-bit read of gfx950 (row pitch 2D + 32 bytes so eight
//     consecutive rows fall on disjoint banks); P enters as a hi + lo pair
//     of bf16 terms so the probabilities keep ~16 significant bits.
// The next tile's K/V loads are issued while the current tile is being
// processed (into the registers the current tile has just released), so
// every wave keeps up to 16 KB in flight with a single register set.
//
// The last tile of a range is masked: tokens at or past the range end
// have their score selected to -inf and their V row zeroed before it
// reaches LDS (the cache may hold NaN there: selection, not
// multiplication, keeps it out).  Block-table entries past the last live
// block are never dereferenced.
//
// 1-byte caches (template KVF: 0 bf16, 1 E4M3FN, 2 uint8 with a zero
// point).  FP8 ([B] "FP8 KV cache"): E4M3FN codes convert exactly to bf16;
// the scale (per block and kv head, per kv head or per tensor: the index
// strides sc_blk / sc_head select it) multiplies the block's scores (K) and
// the block's probabilities before the PV product (V).  INT8 ([B] "INT8 KV
// cache"): code u stands for scale * (u - zp).  With one column tile per
// wave the codes enter the MFMA as the exact bf16 integers u (one
// byte-to-float conversion each) and the zero points are applied outside
// it: a score is scale_k * (q . u - zp_k * sum(q)), and the output
// subtracts sum_t p_t * scale_v * zp_v, accumulated per column beside the
// MFMA sums.  With two column tiles (whose registers are full) the codes
// enter as the exact bf16 integers u - zp instead.
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

#ifndef PKV_WAVES_PER_GROUP
#define PKV_WAVES_PER_GROUP 4
#endif
constexpr int kWavesPerGroup = PKV_WAVES_PER_GROUP;
#ifndef PKV_MIN_WAVES_PER_EU
#define PKV_MIN_WAVES_PER_EU 2
#endif
constexpr int kTile = 32;
// Largest lag (log2 units) of a column's reference max behind its running
// max: probabilities stay <= 2^8, far from fp32 / bf16 overflow.
constexpr float kMaxLag = 8.f;
// SIMDs of an MI355X (256 CUs x 4): the split decode gives each wave two
// consecutive splits when that still leaves one wave per SIMD (measured:
// 1024 longer streams beat 2048 shorter ones by ~2% at 512-token splits)
constexpr long long kSimds = 256LL * 4;

// K/V loads, with or without the non-temporal hint.  A cache much larger
// than the 256 MB MALL is read once per call and should stream (NT = 1):
// as streaming requests the L2 neither stalls on tag allocation nor runs
// out of DRAM request credits (rocprofv3: TCC tag and DRAM-credit stalls
// fall ~60x and the 8B-shape decode runs ~1.9x faster than with
// default-policy loads).  A cache that fits the MALL may be re-read by the
// next call (layers sharing one cache) and keeps the default policy
// (NT = 0), which lets those re-reads hit.
template <int NT>
__device__ __forceinline__ u32x4 load_kv(const unsigned char* p)
{
    if (NT)
        return __builtin_nontemporal_load((const u32x4*)p);
    return *(const u32x4*)p;
}

template <int D, int KVF>
struct Cfg {
    static constexpr int ESZ = KVF ? 1 : 2;            // bytes per cached element
    static constexpr int ROW_BYTES = D * ESZ;           // one token of one kv head
    static constexpr int KSTEPS = D / 32;               // MFMA k-steps of q . k
    static constexpr int K_LOADS = KVF ? D / 64 : D / 32;  // 16-B loads per lane per 16 tokens
    static constexpr int V_LPR = ROW_BYTES / 16;        // lanes per V row
    static constexpr int V_RPI = kWave / V_LPR;         // V rows per load instruction
    static constexpr int V_LOADS = kTile / V_RPI;       // V loads per tile
    static constexpr int DT = D / 16;                   // 16-wide d tiles of the output
    // LDS row pitch of the staged bf16 V rows, bytes: 2D + 32 puts the rows
    // of 8 consecutive tokens on disjoint 8-dword bank ranges (64 banks), so
    // the transposing reads of the PV operands are free of bank conflicts
    static constexpr int PITCH = D * 2 + 32;
    static constexpr int LDS_BYTES = kTile * PITCH;     // per wave
    // LDS row pitch of staged 1-byte K rows (whole-row loads): 16 bytes of
    // padding put the 16 rows one operand read gathers on disjoint banks
    static constexpr int KPITCH = ROW_BYTES + 16;
    static constexpr int Q_BYTES = KSTEPS * kWave * 16;  // Q operands of one column tile
    static_assert(16 % V_RPI == 0, "a V load must stay inside one 16-token block");
};

// LDS slice of one wave: the V staging tile, plus the Q operands when a
// wave has several column tiles (their registers would not fit beside the
// accumulators and the tile in flight; each lane reads back only what it
// wrote, so the slice needs no barrier), plus the K rows when they are
// staged (KROW).
template <int D, int KVF, int NCT, bool KROW = false>
constexpr int wave_lds_bytes()
{
    return Cfg<D, KVF>::LDS_BYTES + (NCT > 1 ? NCT * Cfg<D, KVF>::Q_BYTES : 0)
           + (KROW ? kTile * Cfg<D, KVF>::KPITCH : 0);
}

// First of the 8 consecutive head-dim elements that lane group q feeds to
// MFMA k-step j.  bf16: one 16-byte load per k-step (chunk q + 4j of
// 8 elements).  fp8: one 16-byte load holds two k-steps (chunk q + 4c of
// 16 codes, c = j / 2, low or high half).
template <int KVF>
__device__ __forceinline__ int kdim_base(int j, int q)
{
    return KVF ? 16 * (q + 4 * (j >> 1)) + 8 * (j & 1) : 8 * (q + 4 * j);
}

// Token (within the 32-token tile) held in contraction slot (q, i) of the
// PV product: the S^T output of tile 0 gives lane group q tokens 4q..4q+3,
// tile 1 gives 16+4q..16+4q+3.
__device__ __forceinline__ int pv_token(int q, int i)
{
    return i < 4 ? 4 * q + i : 16 + 4 * q + (i - 4);
}

template <int D, int KVF>
struct Tile {
    u32x4 k[2][Cfg<D, KVF>::K_LOADS];
    u32x4 v[Cfg<D, KVF>::V_LOADS];
};

struct TileAddr {
    int pA, pB;            // physical blocks of tokens 0..15 / 16..31
    float ksA, ksB, vsA, vsB;
    float kzA, kzB, vzA, vzB;   // int8 zero points
};

// 16 cached bytes -> 16 bf16 MFMA operand elements (two 8-element halves):
// fp8 values; int8 codes u (zero point folded out of the MFMA) or u - zp.
template <int KVF, bool FOLD>
__device__ __forceinline__ void codes_to_bf16(u32x4 raw, float zp, u32x4& lo, u32x4& hi)
{
    if (KVF == 1)
        fp8x16_to_bf16x16(raw, lo, hi);
    else
        u8x16_to_bf16x16(raw, FOLD ? 0.f : zp, lo, hi);
}

// Unnormalised result of attending one token range: fp32 accumulators in
// the O^T layout (lane (q, r): O^T[16dt + 4q + i][r]), the running max in
// the exp2 domain and this lane's share of the normaliser.
template <int D>
struct RangeAcc {
    f32x4 acc[D / 16];
    float m;
    float l;
    float corr;     // int8: this lane's share of sum_t p_t * scale_v * zp_v
};

// The MFMA columns of one wave: NCT tiles of 16 columns, each column one
// (query row, query head) pair that reads the wave's kv head.  A decode
// step has one tile whose columns are the G heads of the group; several
// new tokens per sequence give each column its own row and causal limit.
template <int NCT>
struct Cols {
    const uint16_t* qrow[NCT];   // this lane's query vector per column tile
    bool live[NCT];              // the column is a real (row, head) pair
    int lim[NCT];                // causal limit: tokens t < lim are visible
    int mask_from;               // uniform: no column's limit lies below it
};

// Decode columns: column r16 is query head h * G + r16 of sequence b.
__device__ __forceinline__ Cols<1> decode_cols(const DecodeArgs& a, int b, int h, int D)
{
    const int r16 = __lane_id() & 15;
    Cols<1> cs;
    cs.live[0] = r16 < a.G;
    cs.qrow[0] = a.query + ((size_t)b * a.Hq + (cs.live[0] ? h * a.G + r16 : 0)) * D;
    cs.lim[0] = 0x7FFFFFFF;
    cs.mask_from = 0x7FFFFFFF;
    return cs;
}

// The step's new K/V row of (b, h) into the cache slot of position t,
// encoded as paged_kv_append does ([B] "What the KV Cache Stores and Why":
// only the new token's K and V are computed in a decode step); lanes
// 0 .. D/8 - 1 move 8 elements each.
template <int D, int BS, int KVF>
__device__ __forceinline__ void append_row(const DecodeArgs& a, int b, int h, int t)
{
    const int lane = __lane_id();
    if (lane < D / 8) {
        const int p = a.block_tables[(size_t)b * a.max_blocks + t / BS];
        const size_t src = ((size_t)b * a.Hkv + h) * D + 8 * lane;
        const size_t dst = (((size_t)p * BS + t % BS) * a.Hkv + h) * D + 8 * lane;
        store8<KVF>(a.k_new + src, a.v_new + src, (void*)a.k_cache, (void*)a.v_cache, dst,
                    quant_of<KVF>(a.k_scale, a.v_scale, p, h, a.sc_blk, a.sc_head));
    }
}

// Orders this wave's cache stores before its later loads of the same
// slots (other lanes read what a lane wrote).
__device__ __forceinline__ void stores_before_loads()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Segment hook of attend_range: nothing to emit.
struct NoSegments {
    template <int D, int NCT>
    __device__ void operator()(int, RangeAcc<D> (&)[NCT]) const
    {
    }
};

// The block-table entries j_first + lane (j_first: the range's first
// block) when the caller loaded them ahead, beside the sequence length.
struct TableWindow {
    int entries = 0;
    bool loaded = false;
};

// One wave attends its columns (kv head h of sequence b) over the logical
// tokens [t_begin, t_end) (non-empty), streaming 32-token tiles.  With
// CAUSAL, tokens at or past a column's limit are masked as well; a column
// that sees no token of the range ends with l = 0.  append_last: first
// write the step's new row of (b, h) into slot t_end - 1 (the sequence's
// last position), ordered before the loads of the last tile; the wait
// for the stores is placed where the wave waits for its current K tile
// anyway.  seg_tiles > 0: the range is a run of segments of seg_tiles
// tiles (consecutive context splits); at each segment end but the last,
// emit(segment, r) takes the segment's finished state and r restarts,
// while the next segment's first tile is already streaming in.  The last
// segment's state is left in r as for a single range.
template <int D, int BS, int KVF, int NT, int NCT, bool CAUSAL, bool KROW = false,
          typename Emit = NoSegments>
__device__ __forceinline__ void attend_range(const DecodeArgs& a, unsigned char* lds, int b,
                                             int h, int t_begin, int t_end,
                                             const Cols<NCT>& cs, RangeAcc<D> (&r)[NCT],
                                             bool append_last = false, int seg_tiles = 0,
                                             Emit emit = Emit(), TableWindow win = TableWindow())
{
    using C = Cfg<D, KVF>;
    constexpr bool FOLD = KVF == 2 && NCT == 1;   // int8 zero points outside the MFMA
    // KROW (fp8 decode): K is loaded like V, whole rows per lane group (one
    // load instruction covers 8 full 128-byte rows instead of half rows of
    // 16 tokens), staged in LDS as codes and read back in the operand layout
    static_assert(!KROW || (KVF == 1 && NCT == 1 && !CAUSAL), "staged K rows: fp8 decode");
    const int lane = __lane_id();
    const int q4 = lane >> 4;
    const int r16 = lane & 15;
    const int Hkv = a.Hkv;
    if (append_last)
        append_row<D, BS, KVF>(a, b, h, t_end - 1);

    // Q^T operands: column r16 of tile j is this lane's query (zero if
    // dead); in registers for one column tile, in LDS for several.
    constexpr bool QLDS = NCT > 1;
    typedef __attribute__((address_space(3))) volatile u32x4 lds_u32x4;
    lds_u32x4* qlds = (lds_u32x4*)(lds + C::LDS_BYTES);
    bf16x8 qf[QLDS ? 1 : NCT][C::KSTEPS];
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int k = 0; k < C::KSTEPS; ++k) {
            u32x4 v = *(const u32x4*)(cs.qrow[j] + kdim_base<KVF>(k, q4));
            if (!cs.live[j])
                v = u32x4{0u, 0u, 0u, 0u};
            if (QLDS)
                qlds[(j * C::KSTEPS + k) * kWave + lane] = v;
            else
                qf[QLDS ? 0 : j][k] = as_bf16x8(v);
        }
    // int8: sum of each column's query elements (lane groups q4 hold
    // disjoint quarters of the head dimension)
    float qsum[NCT];
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
        qsum[j] = 0.f;
        if (FOLD) {
#pragma unroll
            for (int k = 0; k < C::KSTEPS; ++k) {
                const u32x4 v = *(const u32x4*)(cs.qrow[j] + kdim_base<KVF>(k, q4));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    qsum[j] += bf16_bits_to_f32(v[e] & 0xFFFFu) + bf16_bits_to_f32(v[e] >> 16);
            }
            if (!cs.live[j])
                qsum[j] = 0.f;
            qsum[j] += xor_shuffle(qsum[j], 16);
            qsum[j] += xor_shuffle(qsum[j], 32);
        }
    }
    auto qop = [&](int j, int k) -> bf16x8 {
        if (QLDS) {
            const u32x4 v = qlds[(j * C::KSTEPS + k) * kWave + lane];
            return as_bf16x8(v);
        }
        return qf[QLDS ? 0 : j][k];
    };

    // Block-table window of this unit, 64 entries per VGPR load.
    const int32_t* trow = a.block_tables + (size_t)b * a.max_blocks;
    const int j_first = t_begin / BS;
    const int j_last = (t_end - 1) / BS;
    int tbl_base = win.loaded ? 0 : -1;
    int tbl = win.entries;
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

    // Addresses: a uniform (scalar) physical-block base plus a per-lane
    // 32-bit offset that is the same for every tile.
    const unsigned char* kc = (const unsigned char*)a.k_cache;
    const unsigned char* vc = (const unsigned char*)a.v_cache;
    const uint32_t tok_stride = (uint32_t)Hkv * C::ROW_BYTES;
    const size_t blk_stride = (size_t)BS * tok_stride;
    const uint32_t head_off = (uint32_t)h * C::ROW_BYTES;
    uint32_t k_off[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
        k_off[tau] = (uint32_t)(BS == 16 ? r16 : 16 * tau + r16) * tok_stride + head_off
                     + 16 * q4;
    uint32_t v_off[C::V_LOADS];
#pragma unroll
    for (int k = 0; k < C::V_LOADS; ++k) {
        const int rr = k * C::V_RPI + lane / C::V_LPR;
        v_off[k] = (uint32_t)(BS == 16 ? (rr & 15) : rr) * tok_stride + head_off
                   + 16 * (lane % C::V_LPR);
    }

    // byte offsets of this lane's transposing V^T reads in the staged tile
    const uint32_t tr_off0 = (uint32_t)pv_token(q4, r16 >> 2) * C::PITCH + 8 * (r16 & 3);
    const uint32_t tr_off1 = (uint32_t)pv_token(q4, 4 + (r16 >> 2)) * C::PITCH + 8 * (r16 & 3);

    // Physical blocks (and fp8 scales) of the tile starting at t0.
    auto tile_addr = [&](int t0) {
        TileAddr ta;
        if (BS == 16) {
            ta.pA = phys(t0 / 16);
            ta.pB = phys(t0 / 16 + 1);
        } else {
            ta.pA = phys(t0 / 32);
            ta.pB = ta.pA;
        }
        if (KVF) {
            const size_t iA = (size_t)ta.pA * a.sc_blk + (size_t)h * a.sc_head;
            const size_t iB = (size_t)ta.pB * a.sc_blk + (size_t)h * a.sc_head;
            ta.ksA = a.k_scale[iA];
            ta.vsA = a.v_scale[iA];
            ta.ksB = a.k_scale[iB];
            ta.vsB = a.v_scale[iB];
            if (KVF == 2) {
                ta.kzA = a.k_scale[iA + 1];
                ta.vzA = a.v_scale[iA + 1];
                ta.kzB = a.k_scale[iB + 1];
                ta.vzB = a.v_scale[iB + 1];
            }
        }
        return ta;
    };
    auto load_k = [&](const TileAddr& ta, Tile<D, KVF>& tl) {
        if (KROW) {
            static_assert(!KROW || C::V_LOADS == 2 * C::K_LOADS, "K rows fill the K registers");
#pragma unroll
            for (int k = 0; k < C::V_LOADS; ++k) {
                const int p = (BS == 16 && k * C::V_RPI >= 16) ? ta.pB : ta.pA;
                const unsigned char* blk = kc + (size_t)p * blk_stride;
                tl.k[k / C::K_LOADS][k % C::K_LOADS] = load_kv<NT>(blk + v_off[k]);
            }
            return;
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const unsigned char* blk = kc + (size_t)(tau ? ta.pB : ta.pA) * blk_stride;
#pragma unroll
            for (int c = 0; c < C::K_LOADS; ++c)
                tl.k[tau][c] = load_kv<NT>(blk + k_off[tau] + 64 * c);
        }
    };
    // KROW: the K codes of the tile -> LDS rows (pitch KPITCH); the operand
    // reads gather (token 16 tau + r16, 16-byte chunk q4 + 4c)
    unsigned char* const klds = lds + C::LDS_BYTES;
    auto stage_k = [&](const Tile<D, KVF>& tl) {
#pragma unroll
        for (int k = 0; k < C::V_LOADS; ++k) {
            const int rr = k * C::V_RPI + lane / C::V_LPR;
            *(u32x4*)(klds + rr * C::KPITCH + 16 * (lane % C::V_LPR)) =
                tl.k[k / C::K_LOADS][k % C::K_LOADS];
        }
    };
    auto load_v = [&](const TileAddr& ta, Tile<D, KVF>& tl) {
#pragma unroll
        for (int k = 0; k < C::V_LOADS; ++k) {
            const int p = (BS == 16 && k * C::V_RPI >= 16) ? ta.pB : ta.pA;
            const unsigned char* blk = vc + (size_t)p * blk_stride;
            tl.v[k] = load_kv<NT>(blk + v_off[k]);
        }
    };

    auto reset = [&]() {
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
                r[j].acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            r[j].m = -__builtin_inff();
            r[j].l = 0.f;
            r[j].corr = 0.f;
        }
    };
    // int8 zero points: subtract each column's accumulated correction
    auto apply_fold = [&]() {
        if (FOLD) {
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
                float c = r[j].corr;
                c += xor_shuffle(c, 16);
                c += xor_shuffle(c, 32);
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
                    r[j].acc[dt] -= c;
            }
        }
    };
    reset();
    const float sl2 = a.scale_log2;

    // V rows -> LDS as bf16 (zeroed past the range end).
    auto stage_v = [&](int t0, const TileAddr& ta, const Tile<D, KVF>& tl, bool masked) {
#pragma unroll
        for (int k = 0; k < C::V_LOADS; ++k) {
            const int rr = k * C::V_RPI + lane / C::V_LPR;
            const int c = lane % C::V_LPR;
            u32x4 v = tl.v[k];
            const bool dead = masked && t0 + rr >= t_end;
            if (dead)
                v = u32x4{0u, 0u, 0u, 0u};
            if (KVF) {
                u32x4 lo, hi;
                float zp = 0.f;
                if (KVF == 2 && !FOLD)
                    zp = (BS == 16 && k * C::V_RPI >= 16) ? ta.vzB : ta.vzA;
                codes_to_bf16<KVF, FOLD>(v, zp, lo, hi);
                if (KVF == 2 && !FOLD && dead) {
                    lo = u32x4{0u, 0u, 0u, 0u};
                    hi = u32x4{0u, 0u, 0u, 0u};
                }
                u32x2* dst = (u32x2*)(lds + rr * C::PITCH + 32 * c);
                dst[0] = u32x2{lo[0], lo[1]};
                dst[1] = u32x2{lo[2], lo[3]};
                dst[2] = u32x2{hi[0], hi[1]};
                dst[3] = u32x2{hi[2], hi[3]};
            } else {
                u32x2* dst = (u32x2*)(lds + rr * C::PITCH + 16 * c);
                dst[0] = u32x2{v[0], v[1]};
                dst[1] = u32x2{v[2], v[3]};
            }
        }
    };

    // scores S^T[token][column] of the two 16-token halves, every column
    // tile sharing each K operand
    auto qk = [&](const TileAddr& ta, const Tile<D, KVF>& tl, f32x4 (&sacc)[NCT][2]) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
            for (int j = 0; j < NCT; ++j)
                sacc[j][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < C::K_LOADS; ++c) {
                if (KVF) {
                    u32x4 lo, hi;
                    const u32x4 raw =
                        KROW ? *(const u32x4*)(klds + (16 * tau + r16) * C::KPITCH
                                               + 16 * (q4 + 4 * c))
                             : tl.k[tau][c];
                    codes_to_bf16<KVF, FOLD>(raw, tau ? ta.kzB : ta.kzA, lo, hi);
#pragma unroll
                    for (int j = 0; j < NCT; ++j) {
                        sacc[j][tau] = mfma_16x16x32(as_bf16x8(lo), qop(j, 2 * c), sacc[j][tau]);
                        sacc[j][tau] =
                            mfma_16x16x32(as_bf16x8(hi), qop(j, 2 * c + 1), sacc[j][tau]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < NCT; ++j)
                        sacc[j][tau] = mfma_16x16x32(as_bf16x8(tl.k[tau][c]), qop(j, c),
                                                     sacc[j][tau]);
                }
            }
        }
    };

    // online softmax update and O^T += V^T . P^T from the staged V rows
    auto softmax_pv = [&](int t0, const TileAddr& ta, const f32x4 (&sacc)[NCT][2],
                          bool masked) {
        bf16x8 pb[NCT], pb_lo[NCT];
#pragma unroll
        for (int j = 0; j < NCT; ++j) {
            const int lim = CAUSAL ? min(t_end, cs.lim[j]) : t_end;
            // Scores enter relative to the column's reference max m (0 while
            // nothing is visible): s = score * log2(e) - m, one fma each.
            const float m_ref = r[j].m == -__builtin_inff() ? 0.f : r[j].m;
            float s[8];
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const float f = KVF ? sl2 * (tau ? ta.ksB : ta.ksA) : sl2;
                // int8: (acc - zp_k * sum(q)) * f - m
                const float c = FOLD ? (tau ? ta.kzB : ta.kzA) * qsum[j] * f + m_ref : m_ref;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = __builtin_fmaf(sacc[j][tau][i], f, -c);
                    if (masked && t0 + 16 * tau + 4 * q4 + i >= lim)
                        x = -__builtin_inff();
                    s[4 * tau + i] = x;
                }
            }
            float lm = s[0];
#pragma unroll
            for (int i = 1; i < 8; ++i)
                lm = fmaxf(lm, s[i]);
            // The reference may trail the running max by up to kMaxLag (so
            // p <= 2^kMaxLag): the sums are rescaled only on a column's
            // first visible tile or when a tile raises its max by more than
            // that, which in a long range is a handful of tiles.  The
            // decision is taken for the whole wave.
            if (__builtin_amdgcn_ballot_w64(lm > kMaxLag || r[j].m == -__builtin_inff())) {
                float mt = lm;
                mt = fmaxf(mt, xor_shuffle(mt, 16));
                mt = fmaxf(mt, xor_shuffle(mt, 32));
                const float m_new = fmaxf(r[j].m, m_ref + mt);   // -inf: nothing visible yet
                const float m_ref_new = m_new == -__builtin_inff() ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(r[j].m - m_ref_new);
                const float delta = m_ref_new - m_ref;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    s[i] -= delta;
                r[j].m = m_new;
                r[j].l *= alpha;
                r[j].corr *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
                    r[j].acc[dt] *= alpha;
            }
            float p[8];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                p[i] = __builtin_amdgcn_exp2f(s[i]);
                psum += p[i];
            }
            r[j].l += psum;
            if (KVF) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] *= ta.vsA;
                    p[4 + i] *= ta.vsB;
                }
            }
            if (FOLD)
                r[j].corr += ta.vzA * ((p[0] + p[1]) + (p[2] + p[3]))
                             + ta.vzB * ((p[4] + p[5]) + (p[6] + p[7]));
            // P as a two-term bf16 split, p = hi + lo (about 16 significant
            // bits): one bf16 term alone loses too much when V terms cancel.
            u32x4 pw, pr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
                pr[i] = pack_bf16x2(p[2 * i] - bf16_bits_to_f32(pw[i] & 0xFFFFu),
                                    p[2 * i + 1] - bf16_bits_to_f32(pw[i] >> 16));
            }
            pb[j] = as_bf16x8(pw);
            pb_lo[j] = as_bf16x8(pr);
        }

        // V^T operand of d tile dt: lane (q, r) needs V[pv_token(q, i)][16 dt + r],
        // i = 0..7; two transposing reads, lane (q, 4e + k) naming token
        // pv_token(q, e) (then pv_token(q, 4 + e)) at head-dim 16 dt + 4k
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const u32x2 x0 = lds_read_tr16(lds + tr_off0 + 32 * dt);
            const u32x2 x1 = lds_read_tr16(lds + tr_off1 + 32 * dt);
            const u32x4 vw = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
                r[j].acc[dt] = mfma_16x16x32(as_bf16x8(vw), pb[j], r[j].acc[dt]);
                r[j].acc[dt] = mfma_16x16x32(as_bf16x8(vw), pb_lo[j], r[j].acc[dt]);
            }
        }
    };

    // One register set per wave: a tile's V registers are refilled with
    // the next tile as soon as they are staged in LDS, its K registers as
    // soon as the scores are formed; the next tile's 16 KB then stream in
    // while this tile's softmax and PV product run.  Tiles that end at or
    // before every column's limit skip the causal mask.
    const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
    int n_plain = ntiles - 1;
    if (CAUSAL)
        n_plain = max(0, min(n_plain, (min(t_end, cs.mask_from) - t_begin) / kTile));
    Tile<D, KVF> tl;
    TileAddr ta = tile_addr(t_begin);
    if (append_last && ntiles == 1)
        stores_before_loads();
    load_k(ta, tl);
    load_v(ta, tl);
    auto step = [&](int it, bool masked) {
        const int t0 = t_begin + kTile * it;
        const TileAddr tn = tile_addr(t0 + kTile);
        stage_v(t0, ta, tl, false);
        if (KROW)
            stage_k(tl);
        if (append_last && it == ntiles - 2)
            stores_before_loads();             // tile tn holds slot t_end - 1
        load_v(tn, tl);
        if (KROW)
            load_k(tn, tl);
        f32x4 sacc[NCT][2];
        qk(ta, tl, sacc);
        if (!KROW)
            load_k(tn, tl);
        softmax_pv(t0, ta, sacc, masked);
        ta = tn;
        if (seg_tiles > 0 && (it + 1) % seg_tiles == 0) {   // a segment ends here
            apply_fold();
            emit(it / seg_tiles, r);
            reset();
        }
    };
    for (int it = 0; it < n_plain; ++it)
        step(it, false);
    if (CAUSAL)
        for (int it = n_plain; it < ntiles - 1; ++it)
            step(it, true);
    {
        const int t0 = t_begin + kTile * (ntiles - 1);
        stage_v(t0, ta, tl, true);
        if (KROW)
            stage_k(tl);
        f32x4 sacc[NCT][2];
        qk(ta, tl, sacc);
        softmax_pv(t0, ta, sacc, true);
    }
    apply_fold();
}

// Sums the per-lane normalisers of each head column; returns 1/l and the
// natural-log lse of the range.
template <int D>
__device__ __forceinline__ void finish_range(const RangeAcc<D>& r, float& inv, float& lse)
{
    float l = r.l;
    l += xor_shuffle(l, 16);
    l += xor_shuffle(l, 32);
    inv = l > 0.f ? 1.0f / l : 0.f;          // l = 0: nothing visible, output 0
    lse = (r.m + __builtin_log2f(l)) * kLn2;
}

// Writes this lane's normalised output values of its head column.  Plain
// stores also for partials that the next launch reads: they stay in the
// caches for it (split partials written non-temporally made the 32k-token
// step ~1.7% slower).
template <int D>
__device__ __forceinline__ void store_row(float* o, const RangeAcc<D>& r, float inv)
{
    const int q4 = __lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        *(f32x4*)(o + 16 * dt + 4 * q4) = r.acc[dt] * inv;
}

template <int D>
__device__ __forceinline__ void store_empty_row(float* o)
{
    const int q4 = __lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        *(f32x4*)(o + 16 * dt + 4 * q4) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Fixed partition: one wave per (b, h) over the whole context, or per
// (b, h, group of SPW consecutive splits); split s covers
// [s * split_tokens, min(T, (s + 1) * split_tokens)) and leaves its own
// partial.  Fewer, longer streams keep HBM closer to its peak (a plain
// streaming read: 7.0 TB/s from 1024 waves with 8 KB in flight each,
// 6.0-6.8 TB/s from 2048-16384 waves).
template <int D, int BS, int KVF, int NT, bool SPLIT, int SPW>
__global__ __launch_bounds__(kWavesPerGroup * kWave, PKV_MIN_WAVES_PER_EU)
void decode_kernel(const int32_t* pre_lens, const int32_t* pre_tables, int32_t pre_B,
                   int32_t pre_Hkv, int32_t pre_max_blocks, int32_t pre_max_splits,
                   int32_t pre_split_tokens, DecodeArgs a)
{
    // the fields the first loads need, again as leading scalars preloaded in
    // SGPRs: the length and block-table loads wait for no argument fetch
    a.context_lens = pre_lens;
    a.block_tables = pre_tables;
    a.B = pre_B;
    a.Hkv = pre_Hkv;
    a.max_blocks = pre_max_blocks;
    a.max_splits = pre_max_splits;
    a.split_tokens = pre_split_tokens;
    using C = Cfg<D, KVF>;
    static_assert(SPW == 1 || SPLIT, "split groups only on the split partition");
    __shared__ __attribute__((aligned(16))) unsigned char lds_all[kWavesPerGroup * C::LDS_BYTES];

    const int q4 = __lane_id() >> 4;
    const int r16 = __lane_id() & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = blockIdx.x * kWavesPerGroup + wave;
    const int h = unit % a.Hkv;
    int rest = unit / a.Hkv;
    int split0 = 0;
    if (SPLIT) {
        const int groups = (a.max_splits + SPW - 1) / SPW;
        split0 = (rest % groups) * SPW;
        rest /= groups;
    }
    const int b = rest;
    if (b >= a.B)
        return;
    const int T = a.context_lens[b];
    // the block-table window of the wave's first tile, loaded beside the
    // length instead of after it (entries past the live blocks are read,
    // never dereferenced)
    TableWindow win;
    {
        const long long j0 = SPLIT ? (long long)split0 * a.split_tokens / BS : 0;
        const long long idx = j0 + __lane_id();
        win.entries = idx < a.max_blocks ? a.block_tables[(size_t)b * a.max_blocks + idx] : 0;
        win.loaded = true;
    }
    const int hq = h * a.G + r16;
    const bool live_col = r16 < a.G;
    if (!SPLIT && T <= 0) {                   // empty sequence, single pass
        if (live_col) {
            store_empty_row<D>(a.out + ((size_t)b * a.Hq + hq) * D);
            if (a.lse_out && q4 == 0)
                a.lse_out[(size_t)b * a.Hq + hq] = -__builtin_inff();
        }
        return;
    }
    unsigned char* lds = lds_all + wave * C::LDS_BYTES;
    // the partial of split s (normalised output and natural-log lse)
    auto store_split = [&](int split, RangeAcc<D> (&rr)[1]) {
        float inv, lse;
        finish_range<D>(rr[0], inv, lse);
        if (!live_col)
            return;
        const size_t row = ((size_t)b * a.Hq + hq) * a.max_splits + split;
        store_row<D>(a.partial_out + row * D, rr[0], inv);
        if (q4 == 0)
            a.partial_lse[row] = lse;
    };
    if (!SPLIT) {
        RangeAcc<D> r[1];
        attend_range<D, BS, KVF, NT, 1, false>(a, lds, b, h, 0, T, decode_cols(a, b, h, D), r,
                                               a.k_new != nullptr, 0, NoSegments(), win);
        float inv, lse;
        finish_range<D>(r[0], inv, lse);
        if (!live_col)
            return;
        store_row<D>(a.out + ((size_t)b * a.Hq + hq) * D, r[0], inv);
        if (a.lse_out && q4 == 0)
            a.lse_out[(size_t)b * a.Hq + hq] = lse;
        return;
    }
    // SPW consecutive splits in one pass: the stream does not stop at a
    // split boundary (split_tokens is a multiple of the tile when SPW > 1)
    const int t_begin = split0 * a.split_tokens;
    if (split0 >= a.max_splits || t_begin >= T)
        return;
    const int t_end = (int)min((long long)T, (long long)t_begin + (long long)SPW * a.split_tokens);
    RangeAcc<D> r[1];
    auto emit = [&](int seg, RangeAcc<D> (&rr)[1]) { store_split(split0 + seg, rr); };
    attend_range<D, BS, KVF, NT, 1, false>(a, lds, b, h, t_begin, t_end, decode_cols(a, b, h, D),
                                           r, a.k_new != nullptr && t_end == T,
                                           SPW > 1 ? a.split_tokens / kTile : 0, emit, win);
    store_split(split0 + (t_end - 1 - t_begin) / a.split_tokens, r);
}

// ---------------------------------------------------------------- balanced
// Work-balanced partition.  A work-group is a head group: HG waves, one per
// kv head h = hg * HG + i, that walk the same token ranges together, so the
// Hkv rows of every slot of a physical block are streamed at the same time
// (rocprofv3 / timing: spreading the heads of a block over time costs
// 12-16% of bandwidth).  The work of the call is the list of 32-token
// tiles of every (sequence, head group) unit in (b, hg, tile) order;
// work-group r of R takes tiles [r*W/R, (r+1)*W/R), R being the number of
// work-groups the GPU holds at once, so every group streams the same bytes
// whatever the mix of context lengths.  A unit inside one group's range is
// written straight to `out`; a unit cut by range boundaries leaves one
// normalised partial per piece in the workspace (slot 2r for a group's
// first piece, 2r+1 for its last), the group holding its first piece
// records it (CutRecord), and balanced_merge_kernel combines the pieces of
// every recorded unit with the log-sum-exp rule.
//
// Several new tokens per sequence (MQ): the columns of kv head h are the
// pairs (new row i, head g) in the order c = i * G + g, cut into column
// groups of 16 * NCT; a unit is (sequence, head group, column group) and
// covers the whole context, the causal limits masking what each column
// may not see.

constexpr int kMaxHeadGroup = 8;
constexpr int kMaxMqHeadGroup = 4;

__device__ __forceinline__ int tiles_of(int T)
{
    return (T + kTile - 1) / kTile;
}

// Column groups of sequence b per head group: 1 for a decode step,
// ceil(q_b * G / (16 * NCT)) for q_b new tokens.
template <bool MQ, int NCT>
__device__ __forceinline__ int col_groups(const DecodeArgs& a, int b)
{
    if (!MQ)
        return 1;
    const int q = a.query_start[b + 1] - a.query_start[b];
    return (q * a.G + 16 * NCT - 1) / (16 * NCT);
}

// Tiles of all units of sequence b of one head group.
template <bool MQ, int NCT>
__device__ __forceinline__ long long seq_tiles(const DecodeArgs& a, int b)
{
    return (long long)tiles_of(a.context_lens[b]) * col_groups<MQ, NCT>(a, b);
}

template <bool MQ>
__device__ __forceinline__ long long wave_sum_w(long long v)
{
    return MQ ? wave_sum_ll(v) : (long long)wave_sum_i((int)v);
}

// sum over sequences [0, b_end) of seq_tiles (same value in every lane)
template <bool MQ, int NCT>
__device__ __forceinline__ long long tiles_before(const DecodeArgs& a, int b_end)
{
    long long s = 0;
    for (int c = 0; c < b_end; c += kWave) {
        const int b = c + __lane_id();
        s += wave_sum_w<MQ>(b < b_end ? seq_tiles<MQ, NCT>(a, b) : 0);
    }
    return s;
}

// Sequence whose units contain linear tile x of the (b, unit, tile) list
// (ngroups head groups per sequence); returns b and the tiles per head
// group of the sequences before it.
template <bool MQ, int NCT>
__device__ __forceinline__ void locate_tile(const DecodeArgs& a, int ngroups, long long x,
                                            int& b_out, long long& before_out)
{
    long long base = 0;
    for (int c = 0; c < a.B; c += kWave) {
        const int b = c + __lane_id();
        const long long n = b < a.B ? seq_tiles<MQ, NCT>(a, b) : 0;
        const long long incl =
            MQ ? wave_inclusive_scan_ll(n) : (long long)wave_inclusive_scan((int)n);
        const unsigned long long hit = __ballot((base + incl) * ngroups > x);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            b_out = c + l;
            before_out = base + readlane_ll(incl - n, l);
            return;
        }
        base += readlane_ll(incl, kWave - 1);
    }
    b_out = a.B;
    before_out = base;
}

// floor(r * total / R).  Exact while r * total < 2^52 (checked on the
// host): the double quotient of two exactly represented integers cannot
// cross the integer above the true quotient, whose distance is >= 1/R.
// (A 64-bit integer division is a long software sequence on the GPU.)
__device__ __forceinline__ long long range_start(long long r, long long total, long long R)
{
    return (long long)__builtin_floor((double)(r * total) / (double)R);
}

// Work-groups that get a range: every launched one, or one per tile when
// the call has fewer tiles than work-groups, so that no range is empty and
// the merge walks one work-group per piece (a sequence of a few tiles
// spread over hundreds of empty ranges cost the merge ~39 us).
__device__ __forceinline__ long long ranges_of(long long launched, long long total)
{
    return total < 1 ? 1 : (total < launched ? total : launched);
}

// The work-group whose range holds linear tile x.
__device__ __forceinline__ long long range_of(long long x, long long total, long long R)
{
    long long r = (long long)((double)x * (double)R / (double)total);
    while (r + 1 < R && range_start(r + 1, total, R) <= x)
        ++r;
    while (r > 0 && range_start(r, total, R) > x)
        --r;
    return r;
}

// Decode steps over fp8 caches of 32-token blocks read K as whole rows and
// stage it in LDS (attend_range KROW).
template <int KVF, int BS, bool MQ>
constexpr bool kStagedKRows = KVF == 1 && BS == 32 && !MQ;

// Several new tokens over a bf16 cache: at most four-wave groups at one
// wave per SIMD, so a wave may hold 512 registers (its column tiles'
// accumulators, the tile in flight and the softmax state spilled to
// scratch within 256).
template <int D, int BS, int KVF, int NT, int NCT, bool MQ>
__global__ __launch_bounds__((MQ && KVF == 0) ? kMaxMqHeadGroup * kWave : kMaxHeadGroup * kWave,
                             (MQ && KVF == 0) ? 1 : PKV_MIN_WAVES_PER_EU)
void decode_balanced_kernel(const int32_t* pre_lens, const int32_t* pre_qstart, int32_t pre_B,
                            int32_t pre_Hkv, int32_t pre_G, int32_t pre_groups,
                            int32_t pre_split, int32_t pre_hg, DecodeArgs a, BalanceArgs ws)
{
    // the fields the schedule's first steps read, passed again as leading
    // scalars: they arrive preloaded in SGPRs (kernel-argument preload), so
    // the length scan is issued without a kernel-argument fetch before it
    // first memory access of the kernel (batches of up to 64 sequences):
    // each lane's sequence length (and query offsets), from preloaded
    // scalars only, so nothing waits for a kernel-argument fetch before it
    const bool one_scan = pre_B <= kWave;
    const int lane_b = __lane_id();
    const bool lane_live = one_scan && lane_b < pre_B;
    const int T_first = lane_live ? pre_lens[lane_b] : 0;
    const int qs_first = (MQ && lane_live) ? pre_qstart[lane_b] : 0;
    const int qe_first = (MQ && lane_live) ? pre_qstart[lane_b + 1] : 0;
    a.context_lens = pre_lens;
    a.query_start = pre_qstart;
    a.B = pre_B;
    a.Hkv = pre_Hkv;
    a.G = pre_G;
    ws.ngroups_launched = pre_groups;
    ws.head_split = pre_split;
    ws.head_group = pre_hg;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_all[];  // HG slices

    const int q4 = __lane_id() >> 4;
    const int r16 = __lane_id() & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // head within group
    // NS work-groups share each range, work-group hs of them taking kv
    // heads [(u * NS + hs) * HG, +HG) of list unit u: the halves of a token
    // row are then read at the same time by neighbouring work-groups
    const int NS = ws.head_split;
    const long long wg = blockIdx.x;
    const int hs = (int)(wg % NS);
    const long long r = wg / NS;                     // range
    const int HG = ws.head_group;
    const int ngroups = a.Hkv / (HG * NS);           // list units per sequence (x col groups)
    const int G = a.G;
    constexpr int kCols = 16 * NCT;                  // MQ columns per wave
    const int cpw = MQ ? kCols : G;                  // workspace rows per wave
    // Tiles of the call and the sequence b holding the range's first tile
    // (with the tiles of the sequences before it).  Up to 64 sequences: one
    // length (and query count) per lane serves the total, the search and
    // b's length -- two dependent round trips fewer at the start of every
    // work-group than scanning the lengths again.
    long long incl = 0, n_l = 0;
    int T_l = 0, ncg_l = 0;
    long long total;
    if (one_scan) {
        T_l = T_first;
        ncg_l = !lane_live ? 0 : MQ ? ((qe_first - qs_first) * a.G + kCols - 1) / kCols : 1;
        n_l = (long long)tiles_of(T_l) * ncg_l;
        incl = MQ ? wave_inclusive_scan_ll(n_l) : (long long)wave_inclusive_scan((int)n_l);
        total = readlane_ll(incl, kWave - 1) * ngroups;
    } else {
        total = tiles_before<MQ, NCT>(a, a.B) * ngroups;
    }
    const long long R = ranges_of(ws.ngroups_launched / NS, total);
    const long long r0 = range_start(r, total, R);
    const long long r1 = range_start(r + 1, total, R);
    CutRecord cut = {0, total, 0, -1, 0, 0, 0, 0, 0};
    if (r >= R || r0 >= r1) {
        if (threadIdx.x == 0)
            ws.cuts[wg] = cut;
        return;
    }
    int b, T, ncg;
    long long before;
    if (one_scan) {
        // r0 < total: some lane's inclusive count passes it
        b = __builtin_ctzll(__ballot(incl * ngroups > r0));
        before = readlane_ll(incl - n_l, b);
        T = __builtin_amdgcn_readlane(T_l, b);
        ncg = __builtin_amdgcn_readlane(ncg_l, b);
    } else {
        locate_tile<MQ, NCT>(a, ngroups, r0, b, before);
        T = a.context_lens[b];
        ncg = col_groups<MQ, NCT>(a, b);
    }
    int n = tiles_of(T);
    int u = (int)((r0 - before * ngroups) / n);      // unit of b: hg * ncg + cg
    // fp8 decode on 32-token blocks: K rows staged in LDS (16-token blocks:
    // measured flat to -2.6%, the direct operand loads stay)
    constexpr bool KROW = kStagedKRows<KVF, BS, MQ>;
    unsigned char* lds = lds_all + wave * wave_lds_bytes<D, KVF, NCT, KROW>();
    const int rows_per_slot = HG * cpw;
    long long x = r0;
    int piece = 0;
    while (true) {
        const long long ustart = before * ngroups + (long long)u * n;
        const long long uend = ustart + n;
        const long long pend = uend < r1 ? uend : r1;
        const int t_begin = (int)(x - ustart) * kTile;
        const int t_end = min(T, (int)(pend - ustart) * kTile);
        const int hl = MQ ? u / ncg : u;             // head group within the list
        const int cg = MQ ? u - hl * ncg : 0;
        const int hg = hl * NS + hs;
        const int h = hg * HG + wave;
        const bool whole = x == ustart && pend == uend;
        const size_t slot = 2 * (size_t)wg + (piece == 0 ? 0 : 1);
        if (!MQ) {
            RangeAcc<D> acc[1];
            attend_range<D, BS, KVF, NT, 1, false, KROW>(a, lds, b, h, t_begin, t_end,
                                                   decode_cols(a, b, h, D), acc,
                                                   a.k_new != nullptr && pend == uend);
            float inv, lse;
            finish_range<D>(acc[0], inv, lse);
            if (r16 < G) {
                const int hq = h * G + r16;
                if (whole) {
                    store_row<D>(a.out + ((size_t)b * a.Hq + hq) * D, acc[0], inv);
                    if (a.lse_out && q4 == 0)
                        a.lse_out[(size_t)b * a.Hq + hq] = lse;
                } else {
                    const size_t row = slot * rows_per_slot + wave * G + r16;
                    store_row<D>(ws.part_out + row * D, acc[0], inv);
                    if (q4 == 0)
                        ws.part_lse[row] = lse;
                }
            }
        } else {
            const int qs = a.query_start[b];
            const int q = a.query_start[b + 1] - qs;
            Cols<NCT> cs;
            int qrow[NCT], hq[NCT];
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
                const int c = cg * kCols + 16 * j + r16;
                const int i = c / G;
                cs.live[j] = i < q;
                qrow[j] = qs + (cs.live[j] ? i : 0);
                hq[j] = h * G + (c - i * G);
                cs.qrow[j] = a.query + ((size_t)qrow[j] * a.Hq + hq[j]) * D;
                cs.lim[j] = T - q + i + 1;
            }
            cs.mask_from = T - q + (cg * kCols) / G + 1;
            RangeAcc<D> acc[NCT];
            attend_range<D, BS, KVF, NT, NCT, true>(a, lds, b, h, t_begin, t_end, cs, acc);
#pragma unroll
            for (int j = 0; j < NCT; ++j) {
                float inv, lse;
                finish_range<D>(acc[j], inv, lse);
                if (!cs.live[j])
                    continue;
                if (whole) {
                    const size_t orow = (size_t)qrow[j] * a.Hq + hq[j];
                    store_row<D>(a.out + orow * D, acc[j], inv);
                    if (a.lse_out && q4 == 0)
                        a.lse_out[orow] = lse;
                } else {
                    const size_t row = slot * rows_per_slot + wave * kCols + 16 * j + r16;
                    store_row<D>(ws.part_out + row * D, acc[j], inv);
                    if (q4 == 0)
                        ws.part_lse[row] = lse;
                }
            }
        }
        ++piece;
        x = pend;
        if (x >= r1) {
            if (pend < uend && ustart >= r0) {   // this group holds the unit's first piece
                cut.b = b;
                cut.u = u;
                cut.ustart = ustart;
                cut.n = n;
                cut.ncg = ncg;
                cut.rl = range_of(uend - 1, total, R);
                if (MQ) {
                    cut.qs = a.query_start[b];
                    cut.q = a.query_start[b + 1] - cut.qs;
                }
            }
            break;
        }
        if (++u == ngroups * ncg) {     // next sequence with a non-empty unit
            u = 0;
            before += (long long)n * ncg;
            do {
                ++b;
                T = a.context_lens[b];
                n = tiles_of(T);
                ncg = col_groups<MQ, NCT>(a, b);
            } while (n == 0 || ncg == 0);
        }
    }
    if (threadIdx.x == 0)
        ws.cuts[wg] = cut;
}

// Merge of the recorded cut units.  Work-group (r, y) takes the unit that
// work-group r of the main launch recorded and merges kMergeWaves x
// kMergeRows of its rows (row = kv head of the group x column): each wave
// four rows, 16 lanes per row, each lane D / 16 output elements over every
// piece of the unit, so no lane exchanges anything.  (One row per wave
// launched 4x the waves, and most of them only read a record that holds
// no cut: the launch time followed the wave count, 8.4 us for the 70B
// batch and 23 us for its 4-token verification.)  The extra column r = R
// writes out = 0, lse = -inf for the rows of empty sequences (decode step
// only: with several new tokens an empty sequence has no rows).
constexpr int kMergeWaves = 4;
constexpr int kMergeRows = 4;      // rows per wave

template <int D, int NCT, bool MQ>
__global__ __launch_bounds__(kMergeWaves * kWave)
void balanced_merge_kernel(const CutRecord* pre_cuts, int32_t pre_groups, int32_t pre_split,
                           int32_t pre_hg, DecodeArgs a, BalanceArgs ws)
{
    // the record array and the schedule's shape arrive preloaded in SGPRs
    // (leading scalar arguments), so the record read is issued at once
    ws.cuts = const_cast<CutRecord*>(pre_cuts);
    ws.ngroups_launched = pre_groups;
    ws.head_split = pre_split;
    ws.head_group = pre_hg;
    constexpr int kLanes = kWave / kMergeRows;     // lanes per row
    constexpr int kElems = D / kLanes;             // output elements per lane
    constexpr int kVecs = kElems / 4;
    static_assert(kElems % 4 == 0, "whole f32x4 per lane");
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int HG = ws.head_group;
    const int G = a.G;
    constexpr int kCols = 16 * NCT;
    const int cpw = MQ ? kCols : G;
    if ((long long)blockIdx.x == ws.ngroups_launched) {
        if (MQ)
            return;
        for (int b = blockIdx.y; b < a.B; b += gridDim.y) {
            if (a.context_lens[b] > 0)
                continue;
            for (int hq = wave; hq < a.Hq; hq += kMergeWaves) {
                float* o = a.out + ((size_t)b * a.Hq + hq) * D;
                for (int d = lane; d < D; d += kWave)
                    o[d] = 0.f;
                if (a.lse_out && lane == 0)
                    a.lse_out[(size_t)b * a.Hq + hq] = -__builtin_inff();
            }
        }
        return;
    }
    const CutRecord rec = ws.cuts[blockIdx.x];
    const int b = rec.b;
    if (b < 0)
        return;
    // w * cpw + column
    const int in_slot = (blockIdx.y * kMergeWaves + wave) * kMergeRows + lane / kLanes;
    if (in_slot >= HG * cpw)
        return;
    const int NS = ws.head_split;
    const int hs = (int)(blockIdx.x % NS);           // record of work-group blockIdx.x
    const int u = rec.u;
    const int hl = MQ ? u / rec.ncg : u;
    const int cg = MQ ? u - hl * rec.ncg : 0;
    const int h = (hl * NS + hs) * HG + in_slot / cpw;
    const int cc = in_slot % cpw;
    size_t orow;
    if (!MQ) {
        if (cc >= G)
            return;
        orow = (size_t)b * a.Hq + h * G + cc;
    } else {
        const int col = cg * kCols + cc;
        const int i = col / G;
        if (i >= rec.q)
            return;
        orow = (size_t)(rec.qs + i) * a.Hq + h * G + (col - i * G);
    }
    const int e0 = (lane % kLanes) * kElems;         // this lane's first element
    float* o = a.out + orow * D + e0;
    const long long total = rec.total;
    const long long R = ranges_of(ws.ngroups_launched / NS, total);
    const long long ustart = rec.ustart;
    const long long rf = blockIdx.x / NS;             // range holding the first piece
    const long long rl = rec.rl;
    const int rows_per_slot = HG * cpw;
    // Groups between rf and rl with an empty range (fewer tiles than
    // groups) hold no piece of this unit.
    auto piece_row = [&](long long r) -> long long {
        const long long s0 = range_start(r, total, R);
        if (range_start(r + 1, total, R) <= s0)
            return -1;
        const long long slot = 2 * (r * NS + hs) + ((r == rf && s0 < ustart) ? 1 : 0);
        return slot * rows_per_slot + in_slot;
    };
    // one online pass (running max, rescaled sums) over the pieces, eight
    // pieces' loads in flight per step
    constexpr int kBatch = 8;
    float m = -__builtin_inff();
    float wsum = 0.f;
    f32x4 acc[kVecs];
#pragma unroll
    for (int e = 0; e < kVecs; ++e)
        acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (long long base = rf; base <= rl; base += kBatch) {
        float l[kBatch];
        f32x4 v[kBatch][kVecs];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const long long pr = base + k <= rl ? piece_row(base + k) : -1;
            l[k] = -__builtin_inff();
#pragma unroll
            for (int e = 0; e < kVecs; ++e)
                v[k][e] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (pr >= 0) {
                l[k] = ws.part_lse[pr];
#pragma unroll
                for (int e = 0; e < kVecs; ++e)
                    v[k][e] = *(const f32x4*)(ws.part_out + pr * D + e0 + 4 * e);
            }
        }
        float mb = l[0];
#pragma unroll
        for (int k = 1; k < kBatch; ++k)
            mb = fmaxf(mb, l[k]);
        const float m_new = fmaxf(m, mb);
        if (m_new == -__builtin_inff())
            continue;
        const float sc = __expf(m - m_new);
        wsum *= sc;
#pragma unroll
        for (int e = 0; e < kVecs; ++e)
            acc[e] *= sc;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const float wt = __expf(l[k] - m_new);
            wsum += wt;
#pragma unroll
            for (int e = 0; e < kVecs; ++e)
                acc[e] += wt * v[k][e];
        }
        m = m_new;
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int e = 0; e < kVecs; ++e)
        *(f32x4*)(o + 4 * e) = acc[e] * inv;
    if (a.lse_out && e0 == 0)
        a.lse_out[orow] = m + __logf(wsum);
}

template <int D, int BS, int KVF, int NCT, bool MQ>
int balanced_occupancy(int head_group)
{
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks,
            reinterpret_cast<const void*>(&decode_balanced_kernel<D, BS, KVF, 1, NCT, MQ>),
            head_group * kWave,
            (size_t)head_group * wave_lds_bytes<D, KVF, NCT, kStagedKRows<KVF, BS, MQ>>())
        != hipSuccess)
        return 0;
    return blocks;
}

template <int D, int BS, int KVF, int NCT, bool MQ>
hipError_t launch_balanced_t(const DecodeArgs& a, const BalanceArgs& ws, bool nt,
                             hipStream_t stream)
{
    const size_t lds =
        (size_t)ws.head_group * wave_lds_bytes<D, KVF, NCT, kStagedKRows<KVF, BS, MQ>>();
    const dim3 grid((unsigned)ws.ngroups_launched), block(ws.head_group * kWave);
    if (nt)
        hipLaunchKernelGGL((decode_balanced_kernel<D, BS, KVF, 1, NCT, MQ>), grid, block, lds,
                           stream, a.context_lens, a.query_start, a.B, a.Hkv, a.G,
                           ws.ngroups_launched, ws.head_split, ws.head_group, a, ws);
    else
        hipLaunchKernelGGL((decode_balanced_kernel<D, BS, KVF, 0, NCT, MQ>), grid, block, lds,
                           stream, a.context_lens, a.query_start, a.B, a.Hkv, a.G,
                           ws.ngroups_launched, ws.head_split, ws.head_group, a, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int cpw = MQ ? 16 * NCT : a.G;
    const int rows_per_group = kMergeWaves * kMergeRows;
    const unsigned ychunks = (unsigned)((ws.head_group * cpw + rows_per_group - 1) / rows_per_group);
    const dim3 mgrid((unsigned)ws.ngroups_launched + 1, ychunks);
    hipLaunchKernelGGL((balanced_merge_kernel<D, NCT, MQ>), mgrid, dim3(kMergeWaves * kWave), 0,
                       stream, (const CutRecord*)ws.cuts, ws.ngroups_launched, ws.head_split,
                       ws.head_group, a, ws);
    return hipGetLastError();
}

template <int D, int BS, int KVF, int NT>
hipError_t launch_fixed_t(const DecodeArgs& a, hipStream_t stream)
{
    const bool split = a.split_tokens > 0;
    const long long splits = (long long)a.B * a.Hkv * (split ? a.max_splits : 1);
    // two consecutive splits per wave while that still leaves a wave per SIMD
    const int spw =
        (split && splits >= 2 * kSimds && a.split_tokens % kTile == 0) ? 2 : 1;
    const long long units = (long long)a.B * a.Hkv * (split ? (a.max_splits + spw - 1) / spw : 1);
    const long long groups = (units + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups <= 0)
        return hipSuccess;
    if (groups > 0x7FFFFFFFLL)
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)groups), block(kWavesPerGroup * kWave);
    if (split && spw == 2)
        hipLaunchKernelGGL((decode_kernel<D, BS, KVF, NT, true, 2>), grid, block, 0, stream, a.context_lens,
                           a.block_tables, a.B, a.Hkv, a.max_blocks, a.max_splits,
                           a.split_tokens, a);
    else if (split)
        hipLaunchKernelGGL((decode_kernel<D, BS, KVF, NT, true, 1>), grid, block, 0, stream, a.context_lens,
                           a.block_tables, a.B, a.Hkv, a.max_blocks, a.max_splits,
                           a.split_tokens, a);
    else
        hipLaunchKernelGGL((decode_kernel<D, BS, KVF, NT, false, 1>), grid, block, 0, stream, a.context_lens,
                           a.block_tables, a.B, a.Hkv, a.max_blocks, a.max_splits,
                           a.split_tokens, a);
    return hipGetLastError();
}

template <int D, int BS, int KVF>
hipError_t launch_fixed_d_bs_dt(const DecodeArgs& a, bool nt, hipStream_t stream)
{
    return nt ? launch_fixed_t<D, BS, KVF, 1>(a, stream) : launch_fixed_t<D, BS, KVF, 0>(a, stream);
}

} // namespace

bool balanced_one_group_per_cu(int Hkv, int nct, int kvf)
{
    // Decode of bf16 or fp8 caches: four kv heads per work-group and one
    // work-group per CU, i.e. one wave per SIMD -- fewer, longer HBM
    // streams; measured 4-14% faster than eight-head groups at two per CU
    // (bf16: 70B ragged, 8B, 32k; fp8: 8B and the 36-layer calls; equal
    // on the 70B fp8 batch).  int8 keeps a second wave per SIMD to hide its
    // heavier conversion (9% slower with one on the 70B batch).  Several
    // new tokens over a bf16 cache: four-head groups, one per CU (the
    // kernel's launch bounds give such waves 512 registers; 4-token
    // verification of the 70B batch +15%); the 1-byte formats keep two
    // waves per SIMD (fp8 -6%, int8 -12% with one).
    if (nct > 0)
        return kvf == 0 && Hkv % 4 == 0;
    return kvf != 2 && Hkv % 4 == 0;
}

int balanced_head_group(int Hkv, int nct, int kvf)
{
    if (balanced_one_group_per_cu(Hkv, nct, kvf))
        return 4;
    for (int hg = (nct > 0 && kvf == 0) ? kMaxMqHeadGroup : kMaxHeadGroup; hg > 1; --hg)
        if (Hkv % hg == 0)
            return hg;
    return 1;
}

int balanced_groups_per_cu(int D, int block_size, int kv_dtype, int head_group)
{
#define PKV_OCC(d, bs)                                                                  \
    if (D == d && block_size == bs)                                                    \
        return kv_dtype == 2   ? balanced_occupancy<d, bs, 2, 1, false>(head_group)    \
               : kv_dtype == 1 ? balanced_occupancy<d, bs, 1, 1, false>(head_group)    \
                               : balanced_occupancy<d, bs, 0, 1, false>(head_group);
    PKV_OCC(128, 16)
    PKV_OCC(128, 32)
    PKV_OCC(64, 16)
    PKV_OCC(64, 32)
#undef PKV_OCC
    return 0;
}

hipError_t launch_decode_balanced(const DecodeArgs& a, const BalanceArgs& ws, int D,
                                  int block_size, int kv_dtype, bool nt, hipStream_t stream)
{
#define PKV_BAL(d, bs)                                                                  \
    if (D == d && block_size == bs)                                                    \
        return kv_dtype == 2   ? launch_balanced_t<d, bs, 2, 1, false>(a, ws, nt, stream) \
               : kv_dtype == 1 ? launch_balanced_t<d, bs, 1, 1, false>(a, ws, nt, stream) \
                               : launch_balanced_t<d, bs, 0, 1, false>(a, ws, nt, stream);
    PKV_BAL(128, 16)
    PKV_BAL(128, 32)
    PKV_BAL(64, 16)
    PKV_BAL(64, 32)
#undef PKV_BAL
    return hipErrorInvalidValue;
}

int multiquery_groups_per_cu(int D, int block_size, int kv_dtype, int head_group, int nct)
{
#define PKV_MQOCC(d, bs, n)                                                             \
    if (D == d && block_size == bs && nct == n)                                        \
        return kv_dtype == 2   ? balanced_occupancy<d, bs, 2, n, true>(head_group)     \
               : kv_dtype == 1 ? balanced_occupancy<d, bs, 1, n, true>(head_group)     \
                               : balanced_occupancy<d, bs, 0, n, true>(head_group);
    PKV_MQOCC(128, 16, 1)
    PKV_MQOCC(128, 32, 1)
    PKV_MQOCC(64, 16, 1)
    PKV_MQOCC(64, 32, 1)
    PKV_MQOCC(128, 16, 2)
    PKV_MQOCC(128, 32, 2)
    PKV_MQOCC(64, 16, 2)
    PKV_MQOCC(64, 32, 2)
#undef PKV_MQOCC
    return 0;
}

hipError_t launch_multiquery(const DecodeArgs& a, const BalanceArgs& ws, int D, int block_size,
                             int kv_dtype, int nct, bool nt, hipStream_t stream)
{
#define PKV_MQ(d, bs, n)                                                                \
    if (D == d && block_size == bs && nct == n)                                        \
        return kv_dtype == 2   ? launch_balanced_t<d, bs, 2, n, true>(a, ws, nt, stream) \
               : kv_dtype == 1 ? launch_balanced_t<d, bs, 1, n, true>(a, ws, nt, stream) \
                               : launch_balanced_t<d, bs, 0, n, true>(a, ws, nt, stream);
    PKV_MQ(128, 16, 1)
    PKV_MQ(128, 32, 1)
    PKV_MQ(64, 16, 1)
    PKV_MQ(64, 32, 1)
    PKV_MQ(128, 16, 2)
    PKV_MQ(128, 32, 2)
    PKV_MQ(64, 16, 2)
    PKV_MQ(64, 32, 2)
#undef PKV_MQ
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int D, int block_size, int kv_dtype, bool nt,
                         hipStream_t stream)
{
#define PKV_FIX(d, bs)                                                                  \
    if (D == d && block_size == bs)                                                    \
        return kv_dtype == 2   ? launch_fixed_d_bs_dt<d, bs, 2>(a, nt, stream)         \
               : kv_dtype == 1 ? launch_fixed_d_bs_dt<d, bs, 1>(a, nt, stream)         \
                               : launch_fixed_d_bs_dt<d, bs, 0>(a, nt, stream);
    PKV_FIX(128, 16)
    PKV_FIX(128, 32)
    PKV_FIX(64, 16)
    PKV_FIX(64, 32)
#undef PKV_FIX
    return hipErrorInvalidValue;
}

} // namespace pkv
