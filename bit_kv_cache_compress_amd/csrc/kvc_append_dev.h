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

// Codes c_e = clamp(rint((x_e - zf) / sf), 0, 15) of NE elements (sf != 0), with the quotient
// correctly rounded as an IEEE binary32 division gives it, packed 8 to a word (element e in
// nibble e mod 8 of word e / 8).  The quotient is first taken as (x - zf) * rcp(sf), within a
// few ulp of the correctly rounded one; rint of the two can only differ when the approximation
// lies within 2^-16 of a half-integer (an ulp near 16 is 2^-20), and then the elements take the
// IEEE division.  x - zf is the binary32 difference either way.  Since |q - rint(q)| <= 1/2,
// that test is max |q - rint(q)| >= 1/2 - 2^-16 over the elements, one compare in all.  Two
// codes are packed as one float c_even + 16 c_odd (exact), converted to an integer once.
template <int NE>
__device__ __forceinline__ void value_codes(const float (&x)[NE], float zf, float sf, uint32_t (&w)[NE / 8])
{
    const float r = __builtin_amdgcn_rcpf(sf);
    float dmax = 0.0f;
#pragma unroll
    for (int q = 0; q < NE / 8; ++q) {
        uint32_t word = 0u;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float q0 = (x[8 * q + e] - zf) * r, q1 = (x[8 * q + e + 1] - zf) * r;
            const float t0 = rintf(q0), t1 = rintf(q1);
            dmax = fmaxf(dmax, fmaxf(fabsf(q0 - t0), fabsf(q1 - t1)));
            const float pair = fmaf(16.0f, __builtin_amdgcn_fmed3f(t1, 0.0f, 15.0f), __builtin_amdgcn_fmed3f(t0, 0.0f, 15.0f));
            word |= (uint32_t)pair << (4 * e);
        }
        w[q] = word;
    }
    if (dmax >= 0.5f - 0x1p-16f) {
#pragma unroll
        for (int q = 0; q < NE / 8; ++q) {
            uint32_t word = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = rintf((x[8 * q + e] - zf) / sf);
                word |= (uint32_t)fminf(fmaxf(t, 0.0f), 15.0f) << (4 * e);
            }
            w[q] = word;
        }
    }
}

// Value encode of one token-head by 16 lanes (lane i holds dims 8i..8i+7) into its record:
//   scale = fp16((max - min) / 15), zero = fp16(min) per group of Gv dims (binary32 ops),
//   code  = clamp(rint((x - zero) / scale), 0, 15), 0 when scale == 0;
//   byte m of the 64 code bytes holds dim 2m in its low nibble, dim 2m+1 in its high nibble;
//   the scale/zero words follow the codes.
__device__ __forceinline__ void encode_values(const float (&x)[8], int i, int Gv, uint8_t *rec)
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
    uint32_t word[1] = {0u};
    if (sf != 0.0f) value_codes<8>(x, zf, sf, word);
    reinterpret_cast<uint32_t *>(codes)[i] = word[0];
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
// 4 lanes per token-head (lane j holds dims 32 j .. 32 j + 31), 64 token-heads per 256-thread
// block.  The token-heads are taken head by head: n = (b * Hkv + h) * n_new + t, so that the
// 16 token-heads of a wave are consecutive tokens of one head, whose records are consecutive
// slots of a page: every record is written whole, by full 16-byte stores where it allows.
// ---------------------------------------------------------------------------------------
// v of lane (this lane XOR 1) and (this lane XOR 2) within the quad (DPP quad_perm), for a
// binary64 value.
__device__ __forceinline__ double quad_xor1(double v)
{
    const long long x = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp((int)(x >> 32), 0xB1, 0xF, 0xF, true);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double quad_xor2(double v)
{
    const long long x = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp((int)(x >> 32), 0x4E, 0xF, 0xF, true);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ float quad_xor1f(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Value encode of one token-head by 4 lanes (lane j holds dims 32 j .. 32 j + 31), with the
// arithmetic of encode_values: per group of Gv dims, scale = fp16((max - min) / 15) and
// zero = fp16(min) (binary32 ops), code = clamp(rint((x - zero) / scale), 0, 15) (0 when
// scale == 0); lane j writes bytes 16 j .. 16 j + 15 of the codes and its group's word.
__device__ __forceinline__ void encode_values32(const float (&x)[32], int j, int Gv, uint8_t *rec)
{
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
    if (Gv == 64) {  // two lanes per group
        mn = fminf(mn, quad_xor1f(mn));
        mx = fmaxf(mx, quad_xor1f(mx));
    }
    const float step = (mx - mn) / 15.0f;
    const uint32_t s16 = float_to_half_bits(step);
    const uint32_t z16 = float_to_half_bits(mn);
    const float sf = half_bits_to_float(s16);
    const float zf = half_bits_to_float(z16);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (sf != 0.0f) value_codes<32>(x, zf, sf, w);
    __builtin_memcpy(rec + 16 * j, w, 16);  // 16-byte aligned for Gv 32, 8-byte for Gv 64
    if (Gv == 32 || (j & 1) == 0) reinterpret_cast<uint32_t *>(rec + kD / 2)[(32 * j) / Gv] = s16 | (z16 << 16);
}

__device__ __forceinline__ void append_hadamard_block(const AppendParams &p, long N, long blk)
{
    const int j = threadIdx.x & 3;
    const long n = blk * 64 + (threadIdx.x >> 2);
    if (n >= N) return;  // whole quads exit together: the DPP partners are in the quad
    const int t = (int)(n % p.n_new);
    const long bh = n / p.n_new;
    const int h = (int)(bh % p.c.Hkv), b = (int)(bh / p.c.Hkv);
    const size_t row = ((size_t)((long)b * p.n_new + t) * p.c.Hkv + h) * kD + 32 * j;
    const int pos = p.start_pos[b] + t;
    const int page = p.page_table[(size_t)b * p.max_pages + (pos >> p.c.logP)];
    const size_t slot = ((size_t)page * p.c.Hkv + h) * p.c.P + (pos & (p.c.P - 1));
    // the key's and the value's raw inputs are loaded together, so that the token-head costs
    // one round of memory latency (binary16: 64 bytes of each per lane; binary32 inputs are
    // loaded where they are used).  The value is encoded first, so that its raw words are not
    // held through the key's rotation.
    uint4 kraw[4], vraw[4];
    if (p.dtype == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            kraw[q] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.k) + row + 8 * q);
            vraw[q] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.v) + row + 8 * q);
        }
    }
    float x[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (p.dtype == 0) {
            const uint32_t w[4] = {vraw[q].x, vraw[q].y, vraw[q].z, vraw[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * q + 2 * e] = half_bits_to_float(w[e] & 0xFFFFu);
                x[8 * q + 2 * e + 1] = half_bits_to_float(w[e] >> 16);
            }
        } else {
            float x8[8];
            load8(p.v, p.dtype, row + 8 * q, x8);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * q + e] = x8[e];
        }
    }
    encode_values32(x, j, p.c.Gv, val_rec(p.c, slot));
    __builtin_amdgcn_sched_barrier(0);  // the value's registers are free before the key's rotation
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float x8[8];
        if (p.dtype == 0) {
            const uint32_t w[4] = {kraw[q].x, kraw[q].y, kraw[q].z, kraw[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x8[2 * e] = half_bits_to_float(w[e] & 0xFFFFu);
                x8[2 * e + 1] = half_bits_to_float(w[e] >> 16);
            }
        } else {
            load8(p.k, p.dtype, row + 8 * q, x8);
        }
        if (p.c.kf16) store_key16(p.c, slot, 4 * j + q, x8);
        center8(p.c, h, 4 * j + q, x8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * q + e] = x8[e];
    }
    // sigma, then the 7 butterfly levels (h = 1 .. 16 inside the lane, 32 and 64 across the quad)
    const uint32_t sgw = reinterpret_cast<const uint32_t *>(p.rot)[j];
    double y[32];
    double ss = 0.0;
    // (|k|^2 from the signed copies, y^2 = x^2, so that the binary32 inputs are dead once
    // converted; the chain completes before the butterflies overwrite y)
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const double xe = (double)x[e];
        y[e] = ((sgw >> e) & 1u) ? -xe : xe;
        ss = fma(y[e], y[e], ss);
    }
    ss += quad_xor1(ss);
    ss += quad_xor2(ss);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 32; ++e)
            if ((e & m) == 0) {
                const double a = y[e], c = y[e + m];
                y[e] = a + c;
                y[e + m] = a - c;
            }
        __builtin_amdgcn_sched_barrier(0);  // one level at a time: its inputs die as it goes
    }
    // across the quad: the lane holding the upper index keeps o - y, the other y + o, as one
    // fma with a factor of -1 or +1 (exact)
    const double f1 = (j & 1) ? -1.0 : 1.0, f2 = (j & 2) ? -1.0 : 1.0;
    // (in groups of 8 values, so that the partners' copies do not all live at once)
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        y[e] = fma(f1, y[e], quad_xor1(y[e]));
        if ((e & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        y[e] = fma(f2, y[e], quad_xor2(y[e]));
        if ((e & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    // sign bits: word j of the key record; sum |k'| over the sketch's dims
    uint32_t word = 0;
    double sabs = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        word |= (y[e] < 0.0 ? 0u : 1u) << e;
        sabs += fabs(y[e]);
    }
    if (32 * j >= p.c.sk) sabs = 0.0;  // dims past the sketch
    sabs += quad_xor1(sabs);
    sabs += quad_xor2(sabs);
    sabs /= sqrt((double)kD);  // sum |k'| with k' = y / sqrt(D)
    uint32_t *kr = key_rec(p.c, slot);
    if (j < p.c.kw) kr[j] = word;  // the sketch's words
    if (j == 0) kr[p.c.kw] = norm_corr_word(ss, sabs, p.c.sk);
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
