// pkv_device.hpp -- device-side helpers shared by the gfx950 kernels of
// libpagedkv.so (bf16 / fp8 conversions, MFMA and cross-lane wrappers).
//
// Pages cited: [B] "KV Cache Engineering: PagedAttention, Continuous
// Batching, Attention Variants, and the Bandwidth Wall".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16x16x32 bf16 matrix-core product, fp32 accumulate.  Operand layout on
// a 64-lane wave (q = lane / 16, r = lane % 16):
//   A (16 x 32): lane holds A[r][k] for its 8 k-slots of group q
//   B (32 x 16): lane holds B[k][r] for the same 8 k-slots of group q
//   C (16 x 16): lane holds C[4q + i][r], i = 0..3
// The contraction pairs A's and B's element i of lane group q, so any
// assignment of the 32 contraction indices to (q, i) slots works as long
// as A and B use the same one.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

// Two OCP E4M3FN codes (bytes 2*HI, 2*HI+1 of w) -> two bf16, exact:
// every E4M3FN value, subnormals included, is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 16 fp8 codes (one 16-byte load) -> 16 bf16 (two 8-element operands).
__device__ __forceinline__ void fp8x16_to_bf16x16(u32x4 codes, u32x4& lo, u32x4& hi)
{
    lo[0] = fp8x2_to_bf16x2<false>(codes[0]);
    lo[1] = fp8x2_to_bf16x2<true>(codes[0]);
    lo[2] = fp8x2_to_bf16x2<false>(codes[1]);
    lo[3] = fp8x2_to_bf16x2<true>(codes[1]);
    hi[0] = fp8x2_to_bf16x2<false>(codes[2]);
    hi[1] = fp8x2_to_bf16x2<true>(codes[2]);
    hi[2] = fp8x2_to_bf16x2<false>(codes[3]);
    hi[3] = fp8x2_to_bf16x2<true>(codes[3]);
}

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// 16 unsigned byte codes u -> 16 bf16 values u - zp, in byte order (low
// half bytes 0-7, high half bytes 8-15).  Exact: zp is integer-valued in
// [0, 255], so u - zp is an integer of magnitude <= 255.
__device__ __forceinline__ void u8x16_to_bf16x16(u32x4 codes, float zp, u32x4& lo, u32x4& hi)
{
    uint32_t o[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t x = codes[w];
        o[2 * w] = pack_bf16x2((float)(x & 0xFFu) - zp, (float)((x >> 8) & 0xFFu) - zp);
        o[2 * w + 1] = pack_bf16x2((float)((x >> 16) & 0xFFu) - zp, (float)(x >> 24) - zp);
    }
    lo = u32x4{o[0], o[1], o[2], o[3]};
    hi = u32x4{o[4], o[5], o[6], o[7]};
}

// Transposing LDS read of 16-bit elements (ds_read_b64_tr_b16, gfx950).
// Each lane names 8 bytes (4 elements); inside every group of 16 lanes,
// lane r receives as its element e the element r % 4 of what lane
// 4e + r / 4 of the group named (layout checked on the device).  So if
// lane 4e + k names row e of a matrix at column 4k, lane r gets column r
// of rows 0..3: four rows read across sixteen columns come back as a
// matrix-core operand holding four rows of one column per lane.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* lds_ptr)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_u8*)lds_ptr);
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// Butterfly exchange across lanes (lane ^ mask) through ds_bpermute.
__device__ __forceinline__ float xor_shuffle(float v, int mask)
{
    int lane = __lane_id();
    int src = (lane ^ mask) << 2;
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ int xor_shuffle_i(int v, int mask)
{
    int lane = __lane_id();
    return __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, v);
}

// Value of lane (lane - delta), or 0 for the first `delta` lanes.
__device__ __forceinline__ int shift_up_i(int v, int delta)
{
    int lane = __lane_id();
    int r = __builtin_amdgcn_ds_bpermute((lane - delta) << 2, v);
    return lane >= delta ? r : 0;
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1)
        v += shift_up_i(v, d);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += xor_shuffle_i(v, m);
    return v;
}

// 64-bit forms of the two helpers above (two 32-bit lane exchanges).
__device__ __forceinline__ long long shift_up_ll(long long v, int delta)
{
    const int lo = shift_up_i((int)(unsigned)(unsigned long long)v, delta);
    const int hi = shift_up_i((int)((unsigned long long)v >> 32), delta);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ long long wave_inclusive_scan_ll(long long v)
{
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1)
        v += shift_up_ll(v, d);
    return v;
}

__device__ __forceinline__ long long wave_sum_ll(long long v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const int lo = xor_shuffle_i((int)(unsigned)(unsigned long long)v, m);
        const int hi = xor_shuffle_i((int)((unsigned long long)v >> 32), m);
        v += (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
    }
    return v;
}

__device__ __forceinline__ long long readlane_ll(long long v, int l)
{
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(unsigned long long)v, l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)((unsigned long long)v >> 32), l);
    return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, xor_shuffle(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += xor_shuffle(v, m);
    return v;
}

// binary32 -> OCP E4M3FN, round to nearest even, saturating to +-448,
// NaN -> 0x7F.  Normal results keep the top 3 mantissa bits with an
// integer round-half-even on the 20 dropped bits and rebias the exponent
// (127 -> 7); results below 2^-6 are multiples of 2^-9, obtained as
// rint(|y| * 512) (exact scaling, hardware round-half-even).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float y)
{
    uint32_t u = __builtin_bit_cast(uint32_t, y);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return 0x7Fu;                           // NaN
    if (a >= 0x43E00000u)
        return sign | 0x7Eu;                    // |y| >= 448 (and inf)
    if (a >= 0x3C800000u) {                     // |y| >= 2^-6: normal code
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        return sign | (r - (120u << 3));
    }
    float m = __builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    return sign | (uint32_t)m;                  // 0..8 (8 == smallest normal)
}

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

} // namespace pkv
