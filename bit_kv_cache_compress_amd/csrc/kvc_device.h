// Device-side helpers shared by the gfx950 kernels of libkvcompress.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kD = 128;            // head_dim handled by the kernels
constexpr int kKeyWords = kD / 32;  // 32-bit words of sign bits per key
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
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Lanes below this one in the wave.
__device__ __forceinline__ uint64_t lanemask_lt()
{
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------------------------------
// Top-p bin of a proxy score: floor(s * kbin) in binary32, clamped to [-2^29, 2^29];
// a NaN goes to the bottom.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int score_bin(float s, float kbin)
{
    float x = s * kbin;
    if (!(x >= -(float)kBinClamp)) return -kBinClamp;
    if (x >= (float)kBinClamp) return kBinClamp;
    return (int)floorf(x);
}

// ---------------------------------------------------------------------------------------
// Encoded query of up to GB heads that share one KV head: 4 bit-planes x 4 words of the
// int4 codes per head, c0 = v_l/sqrt(D), c1 = delta/sqrt(D), and the code sum.
// ---------------------------------------------------------------------------------------
template <int GB>
struct QueryState {
    uint32_t plane[GB][4][kKeyWords];
    float c0[GB], c1[GB];
    int sumu[GB];
};

// qpl: [B*Hq][16] words (plane-major), qpar: [B*Hq][4] = (c0, c1, sumu bits, 0).
template <int GB>
__device__ __forceinline__ void load_query(QueryState<GB> &qs, const uint32_t *__restrict__ qpl,
                                           const float4 *__restrict__ qpar, int bh0)
{
#pragma unroll
    for (int h = 0; h < GB; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int w = 0; w < kKeyWords; ++w) qs.plane[h][j][w] = qpl[(bh0 + h) * 16 + j * 4 + w];
        float4 p = qpar[bh0 + h];
        qs.c0[h] = p.x;
        qs.c1[h] = p.y;
        qs.sumu[h] = __float_as_int(p.z);
    }
}

// Proxy score of one cached key against GB query heads (binary x INT4, then the binary32
// combine):  A = 2 * sum_j 2^j popcount(bits & plane_j) - sumu  (= sum_r s_r u_r),
// P = 2 * popcount(bits) - D  (= sum_r s_r),  score = fmaf(c1, A, c0 * P) * (norm / corr).
template <int GB>
__device__ __forceinline__ void score_key(const uint4 kb, uint32_t nc, const QueryState<GB> &qs,
                                          float *s, int *A)
{
    const uint32_t w[4] = {kb.x, kb.y, kb.z, kb.w};
    const int pc = __builtin_popcount(w[0]) + __builtin_popcount(w[1]) + __builtin_popcount(w[2]) +
                   __builtin_popcount(w[3]);
    const float fP = (float)(2 * pc - kD);
    const float r = half_bits_to_float(nc & 0xFFFFu) / half_bits_to_float(nc >> 16);
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        int ip = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int t = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) t += __builtin_popcount(w[q] & qs.plane[h][j][q]);
            ip += t << j;
        }
        const int a = 2 * ip - qs.sumu[h];
        A[h] = a;
        const float cp = qs.c0[h] * fP;
        s[h] = fmaf(qs.c1[h], (float)a, cp) * r;
    }
}

}  // namespace kvc
