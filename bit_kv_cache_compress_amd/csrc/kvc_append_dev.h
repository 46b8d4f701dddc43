// Device code of the appends that both the append kernels and the decode's fused
// query-preparation launch run: the per-token-head encoders for the randomized Hadamard
// rotation and for the dense rotation of a few tokens, and their helpers.
//
// Method: "H1B-KV" (key design: 1-bit key sketch by random projection, 4-bit linear value
// quantization) with the randomized rotation of "RaBitQCache" (abstract).
#pragma once
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

// Eight consecutive input elements of a row, widened to float.
__device__ __forceinline__ void load8(const void *base, int dtype, size_t elem, float x[8])
{
    if (dtype == 0) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = half_bits_to_float(w[e] & 0xFFFFu);
            x[2 * e + 1] = half_bits_to_float(w[e] >> 16);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + elem);
        const float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// Physical slot of token-head n = (b * n_new + t) * Hkv + h.
__device__ __forceinline__ size_t slot_of(const AppendParams &p, long n)
{
    const int h = (int)(n % p.c.Hkv);
    const long bt = n / p.c.Hkv;
    const int t = (int)(bt % p.n_new);
    const int b = (int)(bt / p.n_new);
    const int pos = p.start_pos[b] + t;
    const int page = p.page_table[(size_t)b * p.max_pages + (pos >> p.c.logP)];
    return ((size_t)page * p.c.Hkv + h) * p.c.P + (pos & (p.c.P - 1));
}

// Value encode of one token-head by 16 lanes (lane i holds dims 8i..8i+7) into its record:
//   scale = fp16((max - min) / 15), zero = fp16(min) per group of Gv dims (binary32 ops),
//   code  = clamp(rint((x - zero) / scale), 0, 15), 0 when scale == 0;
//   byte m of the 64 code bytes holds dim 2m in its low nibble, dim 2m+1 in its high nibble;
//   the scale/zero words follow the codes.
__device__ __forceinline__ void encode_values(const float x[8], int i, int Gv, uint8_t *rec)
{
    uint8_t *codes = rec;
    uint32_t *sz = reinterpret_cast<uint32_t *>(rec + kD / 2);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
    const int gl = Gv / 8;  // lanes per group
    for (int o = 1; o < gl; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    const float range = mx - mn;
    const float step = range / 15.0f;
    const uint32_t s16 = float_to_half_bits(step);
    const uint32_t z16 = float_to_half_bits(mn);
    const float sf = half_bits_to_float(s16);
    const float zf = half_bits_to_float(z16);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int c = 0;
        if (sf != 0.0f) {
            float t = rintf((x[e] - zf) / sf);
            t = fminf(fmaxf(t, 0.0f), 15.0f);
            c = (int)t;
        }
        word |= (uint32_t)c << (4 * e);
    }
    reinterpret_cast<uint32_t *>(codes)[i] = word;
    if ((i & (gl - 1)) == 0) sz[(8 * i) / Gv] = s16 | (z16 << 16);
}

// The binary16 copy of key dims 8i .. 8i+7 of a slot (one 16-byte store), for caches that
// keep one: x is the input key widened to binary32, rounded to nearest even.
__device__ __forceinline__ void store_key16(const CacheView &c, size_t slot, int i, const float (&x)[8])
{
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = float_to_half_bits(x[2 * q]) | (float_to_half_bits(x[2 * q + 1]) << 16);
    reinterpret_cast<uint4 *>(c.kf16 + slot * kD)[i] = make_uint4(w[0], w[1], w[2], w[3]);
}

// Key centering: x -= c (binary32) for dims 8i .. 8i+7 of KV head h, when the cache has
// centers; the sign bits, norm and correction are then those of k - c.
__device__ __forceinline__ void center8(const CacheView &c, int h, int i, float (&x)[8])
{
    if (!c.kc) return;
    const float4 *cr = reinterpret_cast<const float4 *>(c.kc + (size_t)h * kD + 8 * i);
    const float4 a = cr[0], b = cr[1];
    x[0] -= a.x; x[1] -= a.y; x[2] -= a.z; x[3] -= a.w;
    x[4] -= b.x; x[5] -= b.y; x[6] -= b.z; x[7] -= b.w;
}

// Sum over the 16 lanes of a token-head group.
__device__ __forceinline__ double sum16(double v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// key_nc word: binary16 |k| (low) and binary16 sum_{r<sk} |k'_r| / (sqrt(sk) |k|) (high;
// 1 if k = 0), sk the sketch width (sign bits per key).
__device__ __forceinline__ uint32_t norm_corr_word(double ss, double sabs_rot, int sk)
{
    const double nrm = sqrt(ss);
    const double corr = (nrm == 0.0) ? 1.0 : sabs_rot / (sqrt((double)sk) * nrm);
    return double_to_half_bits(nrm) | (double_to_half_bits(corr) << 16);
}

// ---------------------------------------------------------------------------------------
// Randomized Hadamard rotation: k' = H diag(sigma) k / sqrt(D), in binary64 butterflies.
// 16 lanes per token-head, 16 token-heads per 256-thread block.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void append_hadamard_block(const AppendParams &p, long N, long blk)
{
    const int i = threadIdx.x & 15;
    const long n = blk * 16 + (threadIdx.x >> 4);
    if (n >= N) return;  // whole 16-lane groups exit together
    const size_t row = (size_t)n * kD + 8 * i;
    float xk[8], xv[8];
    load8(p.k, p.dtype, row, xk);
    load8(p.v, p.dtype, row, xv);
    const size_t slot = slot_of(p, n);
    if (p.c.kf16) store_key16(p.c, slot, i, xk);
    center8(p.c, (int)(n % p.c.Hkv), i, xk);

    // sigma, then the 7 butterfly levels (h = 1, 2, 4 inside the lane, 8..64 across lanes)
    const uint32_t sgw = reinterpret_cast<const uint32_t *>(p.rot)[i >> 2];
    double y[8];
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double xe = (double)xk[e];
        ss += xe * xe;
        const int d = 8 * i + e;
        y[e] = ((sgw >> (d & 31)) & 1u) ? -xe : xe;
    }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & h) == 0) {
                const double a = y[e], b = y[e + h];
                y[e] = a + b;
                y[e + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double o = __shfl_xor(y[e], m);
            y[e] = (i & m) ? (o - y[e]) : (y[e] + o);
        }
    // sign bits: byte i of the 16-byte key word vector
    uint32_t byte = 0;
    double sabs = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        byte |= (y[e] < 0.0 ? 0u : 1u) << e;
        sabs += fabs(y[e]);
    }
    uint32_t word = byte << (8 * (i & 3));
    word |= __shfl_xor(word, 1);
    word |= __shfl_xor(word, 2);
    if ((i & 3) == 0 && (i >> 2) < p.c.kw) key_rec(p.c, slot)[i >> 2] = word;  // the sketch's words
    if (8 * i >= p.c.sk) sabs = 0.0;        // dims past the sketch
    ss = sum16(ss);
    sabs = sum16(sabs) / sqrt((double)kD);  // sum |k'| with k' = y / sqrt(D)
    if (i == 0) key_rec(p.c, slot)[p.c.kw] = norm_corr_word(ss, sabs, p.c.sk);
    encode_values(xv, i, p.c.Gv, val_rec(p.c, slot));
}

// ---------------------------------------------------------------------------------------
// Dense rotation for few token-heads (the per-step append of a decode loop): one 256-thread
// block per token-head.  Thread t computes half (t >> 5) & 1 of row 32 (t >> 6) + (t & 31) of
// k' = R k as a binary64 fused chain over 64 columns, and the two halves are added.  Every
// load (the key, the value, the 64 binary16 entries of the row half) is issued at the start,
// so the block costs one round of memory latency plus the 64-step chain.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void append_small_block(const AppendParams &p, long N, long n)
{
    __shared__ double kd[kD];
    __shared__ double red[8];
    __shared__ uint32_t rows[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (n >= N) return;
    const int hc = lane >> 5;
    const int r = 32 * w + (lane & 31);
    const uint4 *Rr = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.rot) + r * kD + 64 * hc);
    uint4 a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = Rr[i];
    float xk[8], xv[8];
    if (t < 16) load8(p.k, p.dtype, (size_t)n * kD + 8 * t, xk);
    if (t >= 64 && t < 80) load8(p.v, p.dtype, (size_t)n * kD + 8 * (t - 64), xv);
    const size_t slot = slot_of(p, n);
    if (t < 16) {
        if (p.c.kf16) store_key16(p.c, slot, t, xk);
        center8(p.c, (int)(n % p.c.Hkv), t, xk);
#pragma unroll
        for (int e = 0; e < 8; ++e) kd[8 * t + e] = (double)xk[e];
    }
    __syncthreads();
    double y = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t wa[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            y = fma((double)half_bits_to_float((wa[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), kd[64 * hc + 8 * i + e], y);
    }
    y += __shfl_xor(y, 32);  // both halves of the row
    const uint64_t m = __ballot(!(y < 0.0));  // bit (lane & 31) = row 32 w + (lane & 31)
    double sabs = hc == 0 ? fabs(y) : 0.0;
    double ss = t < kD ? kd[t] * kd[t] : 0.0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sabs += __shfl_xor(sabs, o);
        ss += __shfl_xor(ss, o);
    }
    if (lane == 0) {
        red[w] = sabs;
        red[4 + w] = ss;
        rows[w] = (uint32_t)m;
    }
    __syncthreads();
    if (t == 0) {
        uint32_t *kr = key_rec(p.c, slot);
        for (int q = 0; q < p.c.kw; ++q) kr[q] = rows[q];  // wave w holds rows 32 w .. 32 w + 31
        const double sabs = p.c.kw == 4 ? (red[0] + red[1]) + (red[2] + red[3]) : red[0] + red[1];
        kr[p.c.kw] = norm_corr_word((red[4] + red[5]) + (red[6] + red[7]), sabs, p.c.sk);
    }
    if (t >= 64 && t < 80)
        encode_values(xv, t - 64, p.c.Gv, val_rec(p.c, slot));
}


}  // namespace kvc
