// Device-side helpers shared by the gfx950 kernels of libkvcompress.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kD = 128;            // head_dim handled by the kernels
constexpr int kBins = 8192;        // Top-p bin distances with non-zero weight
constexpr int kBinClamp = 1 << 29;
constexpr int kBlock = 256;

// ---------------------------------------------------------------------------------------
// binary16 helpers
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    uint16_t b = (uint16_t)bits16;
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}

// float -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t float_to_half_bits(float f)
{
    _Float16 h = (_Float16)f;
    uint16_t b;
    __builtin_memcpy(&b, &h, 2);
    return b;
}

// binary64 -> binary16 bits, correctly rounded.  The binary64 value is first rounded to
// binary32 with round-to-odd (RNE, then step to the odd neighbour toward x when inexact);
// a round-to-odd intermediate with at least two more bits than the target makes the second
// rounding (binary32 -> binary16, RNE) equal to a direct correct rounding.
__device__ __forceinline__ uint32_t double_to_half_bits(double x)
{
    float f = (float)x;
    if ((double)f != x) {
        uint32_t fb = __float_as_uint(f);
        if ((fb & 1u) == 0u) fb = (fabs((double)f) > fabs(x)) ? fb - 1u : fb + 1u;
        f = __uint_as_float(fb);
    }
    return float_to_half_bits(f);
}

// ---------------------------------------------------------------------------------------
// Wave / block reductions (wave64)
// ---------------------------------------------------------------------------------------
// Lane index within the wave (v_mbcnt).
__device__ __forceinline__ int lane_id()
{
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
// v of lane (this lane XOR m), m < 64: one ds_bpermute over the whole wave, without the
// sub-width bound of __shfl_xor (whose wave-constant bound the compiler otherwise keeps
// live, and spills, across long loops).
__device__ __forceinline__ int xor_lane(int v, int m)
{
    return __builtin_amdgcn_ds_bpermute((lane_id() ^ m) << 2, v);
}
__device__ __forceinline__ float xor_lane(float v, int m)
{
    return __int_as_float(xor_lane(__float_as_int(v), m));
}
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, xor_lane(v, o));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, xor_lane(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += xor_lane(v, o);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += xor_lane(v, o);
    return v;
}

// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanemask_lt()
{
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Byte K of x as a float (v_cvt_f32_ubyteK: one instruction, where the compiler would
// otherwise extract the field first).
template <int K>
__device__ __forceinline__ float ubyte_to_float(uint32_t x)
{
    float f;
    if constexpr (K == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(x));
    else if constexpr (K == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
    else if constexpr (K == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(x));
    return f;
}

// The 8 codes of a code word as c * 2^-9, two per instruction: a byte holding a code c < 16,
// read as an OCP E4M3 number (gfx950's fp8), is exactly c * 2^-9 (a subnormal for c < 8, the
// exponent's lowest normal binade for c >= 8), so v_cvt_pk_f32_fp8 converts two codes at once.
// A caller multiplies its weight by 2^9 (exact): w 2^9 * c 2^-9 rounds as w * c does.
constexpr float kCodeUnscale = 512.0f;
__device__ __forceinline__ void unpack_codes_e4m3(uint32_t w, float c[8])
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // dims 0,2,4,6 / 1,3,5,7
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // bytes 0, 1: dims 0, 2
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // bytes 2, 3: dims 4, 6
    const auto x = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);  // dims 1, 3
    const auto y = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);   // dims 5, 7
    c[0] = a[0];
    c[1] = x[0];
    c[2] = a[1];
    c[3] = x[1];
    c[4] = b[0];
    c[5] = y[0];
    c[6] = b[1];
    c[7] = y[1];
}

// The 8 codes of a 32-bit code word (dims 2m in the low, 2m+1 in the high nibble of byte m)
// as floats, c[0..7] in dim order.
__device__ __forceinline__ void unpack_codes(uint32_t w, float c[8])
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    c[0] = ubyte_to_float<0>(lo);
    c[1] = ubyte_to_float<0>(hi);
    c[2] = ubyte_to_float<1>(lo);
    c[3] = ubyte_to_float<1>(hi);
    c[4] = ubyte_to_float<2>(lo);
    c[5] = ubyte_to_float<2>(hi);
    c[6] = ubyte_to_float<3>(lo);
    c[7] = ubyte_to_float<3>(hi);
}

// Sum over the 4 lanes of a quad (DPP quad_perm 1,0,3,2 then 2,3,0,1); every lane gets it.
__device__ __forceinline__ float quad_sum(float v)
{
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    return v;
}

// Wave-wide max, uniform result: DPP within each 16-lane row, then the four row maxima.
// Wave max of an int, returned in a scalar register: DPP within rows, then the 4 row maxima.
__device__ __forceinline__ int wave_max_iu(int v)
{
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true));  // row_ror 4
    v = max(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true));  // row_ror 8
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

__device__ __forceinline__ float wave_max_u(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));   // quad_perm 1,0,3,2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));   // quad_perm 2,3,0,1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true)));  // row_ror 4
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true)));  // row_ror 8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ---------------------------------------------------------------------------------------
// norm / corr of a key record's binary16 pair, rounded to nearest binary32: the same value
// as IEEE division, in fewer instructions.  y = rcp(c) is within one ulp of 1/c, so
// q0 = n * y is within three ulps of q = n / c and the remainder n - c * q0 is exact in one
// fma; q1 = q0 + (n - c q0) * y then differs from q by less than 2^-20 ulp.  A quotient of
// two binary16 numbers lies more than 2^-12 ulp from every rounding midpoint of binary32
// (such a midpoint has an odd 25-bit significand, and its distance to n / c is a nonzero
// multiple of a power of two that c's 11-bit significand bounds), so q1 is rounded as q.
// Where q1 is NaN (a zero, infinite or NaN operand) or zero (n = 0, where the sum with the
// zero remainder can lose the sign of q0), q0 is the IEEE quotient and is taken instead.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float norm_over_corr(uint32_t nc)
{
    const float n = half_bits_to_float(nc & 0xFFFFu), c = half_bits_to_float(nc >> 16);
    const float y = __builtin_amdgcn_rcpf(c);
    const float q0 = n * y;
    const float q1 = fmaf(fmaf(-c, q0, n), y, q0);
    return __builtin_amdgcn_class(q1, 0x63) ? q0 : q1;  // classes sNaN, qNaN, -0, +0
}

// ---------------------------------------------------------------------------------------
// Top-p bin of a proxy score: floor(s * kbin) in binary32, clamped to [-2^29, 2^29];
// a NaN goes to the bottom.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int score_bin(float s, float kbin)
{
    const float x = fminf(fmaxf(s * kbin, -(float)kBinClamp), (float)kBinClamp);  // NaN -> bottom
    int e;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(e) : "v"(x));  // floor, then to int32 (exact here)
    return e;
}

// ---------------------------------------------------------------------------------------
// Encoded query of up to GB heads that share one KV head.  The int4 codes are kept as
// 16 words per head in the order the 8 x 4-bit dot product (v_dot8_u32_u4) consumes them:
// nib[4w + k] holds, in nibble m = 0..7, the code of dim 32w + 4m + k.  A key word w
// spread to nibbles (spread_key) puts twice the sign bit of the same dims in the same
// nibbles, so  sum_{w,k} dot8(spread_key(w, k), nib[4w + k]) = 2 sum_r bit_r u_r.
// c0 = v_l/sqrt(D), c1 = delta/sqrt(D), sumu = sum of the codes.
// ---------------------------------------------------------------------------------------
template <int GB>
struct QueryState {
    uint32_t nib[GB][16];
    float c0[GB], c1[GB];
    int sumu[GB];
};

// Block-wide staging of the GB heads' query state through LDS (qsh: GB*16 words, qps: GB
// float4).  Reading it back from LDS keeps one copy per lane in vector registers; as
// uniform scalar loads the 64 words of 4 heads would overflow the scalar register file.
// Caller synchronizes between stage_query and read_query.
template <int GB>
__device__ __forceinline__ void stage_query(const uint32_t *__restrict__ qnib, const float4 *__restrict__ qpar,
                                            int bh0, uint32_t *qsh, float4 *qps)
{
    const int t = threadIdx.x;
    if (t < GB * 16) qsh[t] = qnib[(size_t)(bh0 + t / 16) * 16 + (t & 15)];
    if (t < GB) qps[t] = qpar[bh0 + t];
}

template <int GB>
__device__ __forceinline__ void read_query(QueryState<GB> &qs, const uint32_t *qsh, const float4 *qps)
{
#pragma unroll
    for (int h = 0; h < GB; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) qs.nib[h][i] = qsh[h * 16 + i];
        const float4 p = qps[h];
        qs.c0[h] = p.x;
        qs.c1[h] = p.y;
        qs.sumu[h] = __float_as_int(p.z);
    }
}

// An integer 0 <= x < 256 with at most 4 significant bits as its fp8 (OCP e4m3) code:
// exponent field floor(log2 x) + 7, the three bits below the leading one as the mantissa.
__device__ __forceinline__ uint32_t fp8_e4m3_small(int x)
{
    if (x == 0) return 0u;
    const int e = 31 - __builtin_clz((uint32_t)x);
    return (uint32_t)(((e + 7) << 3) | (((x << 3) >> e) & 7));
}

// Key word w spread for the dot8 products: nibble m of spread_key(w, k) is 2 * bit (4m + k)
// of w.  With the query word nib[4w + k] this gives 2 * sum_r bit_r u_r.
__device__ __forceinline__ uint32_t spread_key(uint32_t w, int k)
{
    return (k == 0 ? (w << 1) : k == 1 ? w : (w >> (k - 1))) & 0x22222222u;
}

// Proxy score of one cached key against GB query heads (binary x INT4, then the binary32
// combine):  A = 2 * sum_r bit_r u_r - sumu  (= sum_r s_r u_r, s_r = +-1; the dot8 chain
// starts at -sumu and wraps modulo 2^32), P = 2 * popcount(bits) - sk  (= sum_r s_r over the
// sk sketch bits; the words past them are zero, as are the query codes of those dims),
// score = fmaf(c1, A, c0 * P) * (norm / corr).
template <int GB>
__device__ __forceinline__ void score_key(const uint4 kb, uint32_t nc, const QueryState<GB> &qs,
                                          float *s, int *A, int sk)
{
    const uint32_t w[4] = {kb.x, kb.y, kb.z, kb.w};
    uint32_t x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) x[4 * i + k] = spread_key(w[i], k);
    const int pc = __builtin_popcount(w[0]) + __builtin_popcount(w[1]) + __builtin_popcount(w[2]) +
                   __builtin_popcount(w[3]);
    const float fP = (float)(2 * pc - sk);
    const float r = norm_over_corr(nc);
    // the GB accumulation chains are interleaved so that consecutive dot products are
    // independent
    uint32_t ip[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) ip[h] = (uint32_t)(-qs.sumu[h]);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int h = 0; h < GB; ++h) ip[h] = __builtin_amdgcn_udot8(x[i], qs.nib[h][i], ip[h], false);
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        const int a = (int)ip[h];
        A[h] = a;
        const float cp = qs.c0[h] * fP;
        s[h] = fmaf(qs.c1[h], (float)a, cp) * r;
    }
}

}  // namespace kvc
