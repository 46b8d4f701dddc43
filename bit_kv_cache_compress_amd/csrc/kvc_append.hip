// Append kernels: encode new keys (sign bits of a random rotation + binary16 norm and
// correction) and values (per-group 4-bit linear codes) into the paged cache.
//
// Method: "H1B-KV" (key design: 1-bit key sketch by random projection, 4-bit linear value
// quantization) with the randomized rotation of "RaBitQCache" (abstract).  The sign of each
// rotated coordinate is decided on the exact product: for binary16 (and, in practice,
// binary32) inputs every partial sum of R k is exact in binary64, so the kernels rotate in
// binary64 -- a butterfly for the randomized Hadamard rotation and binary64 MFMA for the
// dense one -- and their sign bits do not depend on the summation order.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

typedef double double4_t __attribute__((ext_vector_type(4)));

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

// key_nc word: binary16 |k| (low) and binary16 sum|k'| / (sqrt(D) |k|) (high; 1 if k = 0).
__device__ __forceinline__ uint32_t norm_corr_word(double ss, double sabs_rot)
{
    const double nrm = sqrt(ss);
    const double corr = (nrm == 0.0) ? 1.0 : sabs_rot / (sqrt((double)kD) * nrm);
    return double_to_half_bits(nrm) | (double_to_half_bits(corr) << 16);
}

// ---------------------------------------------------------------------------------------
// Randomized Hadamard rotation: k' = H diag(sigma) k / sqrt(D), in binary64 butterflies.
// 16 lanes per token-head, 16 token-heads per 256-thread block.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_append_hadamard(AppendParams p, long N)
{
    const int i = threadIdx.x & 15;
    const long n = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
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
    if ((i & 3) == 0) key_rec(p.c, slot)[i >> 2] = word;
    ss = sum16(ss);
    sabs = sum16(sabs) / sqrt((double)kD);  // sum |k'| with k' = y / sqrt(D)
    if (i == 0) key_rec(p.c, slot)[kKeyWords] = norm_corr_word(ss, sabs);
    encode_values(xv, i, p.c.Gv, val_rec(p.c, slot));
}

// ---------------------------------------------------------------------------------------
// Dense rotation k' = R k with binary64 MFMA (v_mfma_f64_16x16x4f64): each wave rotates 16
// token-heads (A = 16 keys x 4 dims, B = 4 dims x 16 rows of R^T, 32 steps x 8 row blocks).
// 128-thread blocks, 32 token-heads per tile, R staged once per block in LDS (binary16,
// rows padded to 130 halves so the 16 rows read by one MFMA fall in distinct banks).
// ---------------------------------------------------------------------------------------
constexpr int kRStride = 130;

__global__ __launch_bounds__(128) void k_append_dense(AppendParams p, long N)
{
    __shared__ uint16_t Rs[kD * kRStride];
    __shared__ float Ks[32 * kD];       // key tile widened to float (exact for f16 and f32)
    __shared__ double sabs_s[32];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const uint16_t *R = reinterpret_cast<const uint16_t *>(p.rot);
    for (int c = tid; c < kD * kD / 8; c += 128) {
        const uint4 raw = reinterpret_cast<const uint4 *>(R)[c];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const int r = c >> 4, j0 = (c & 15) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Rs[r * kRStride + j0 + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
            Rs[r * kRStride + j0 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
        }
    }

    const long ntiles = (N + 31) / 32;
    for (long tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        __syncthreads();  // R ready / previous tile finished with Ks, sabs_s
        // stage the key tile: 32 rows x 128 dims, 8 dims per thread-iteration
        for (int c = tid; c < 32 * 16; c += 128) {
            const int r = c >> 4, i = c & 15;
            const long n = tile * 32 + r;
            float x[8];
            if (n < N) {
                load8(p.k, p.dtype, (size_t)n * kD + 8 * i, x);
                if (p.c.kf16) store_key16(p.c, slot_of(p, n), i, x);
                center8(p.c, (int)(n % p.c.Hkv), i, x);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) Ks[r * kD + 8 * i + e] = x[e];
        }
        __syncthreads();

        // MFMA: this wave's 16 rows are tile rows 16*wave .. 16*wave+15
        double4_t acc[8];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) acc[rb] = (double4_t){0.0, 0.0, 0.0, 0.0};
        const int arow = 16 * wave + (lane & 15);
        const int kq = lane >> 4;
        for (int js = 0; js < 32; ++js) {
            const double a = (double)Ks[arow * kD + 4 * js + kq];
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                const double b = (double)half_bits_to_float(Rs[(16 * rb + (lane & 15)) * kRStride + 4 * js + kq]);
                acc[rb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[rb], 0, 0, 0);
            }
        }
        // accumulator v of lane l holds k'[row 4*v + l/16][dim 16*rb + l%16]
        const int q = lane & 3;  // lanes 0..3 assemble rows 4v+q
        uint32_t words[4][4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
            for (int w = 0; w < 4; ++w) words[v][w] = 0u;
            double sa = 0.0;
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                const double val = acc[rb][v];
                sa += fabs(val);
                const uint64_t m = __ballot(!(val < 0.0));
                const uint32_t bits16 = (uint32_t)((m >> (16 * q)) & 0xFFFFull);
                words[v][rb >> 1] |= bits16 << (16 * (rb & 1));
            }
            sa = sum16(sa);
            if ((lane & 15) == 0) sabs_s[16 * wave + 4 * v + (lane >> 4)] = sa;
        }
        if (lane < 4) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const long n = tile * 32 + 16 * wave + 4 * v + q;
                if (n < N) {
                    const size_t slot = slot_of(p, n);
                    uint32_t *kr = key_rec(p.c, slot);
#pragma unroll
                    for (int q2 = 0; q2 < kKeyWords; ++q2) kr[q2] = words[v][q2];
                }
            }
        }
        __syncthreads();

        // norms, corrections and values: 16 lanes per token-head, 8 token-heads per pass
        for (int pass = 0; pass < 4; ++pass) {
            const int r = pass * 8 + (tid >> 4);
            const int i = tid & 15;
            const long n = tile * 32 + r;
            if (n < N) {
                double ss = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double xe = (double)Ks[r * kD + 8 * i + e];
                    ss += xe * xe;
                }
                ss = sum16(ss);
                const size_t slot = slot_of(p, n);
                if (i == 0) key_rec(p.c, slot)[kKeyWords] = norm_corr_word(ss, sabs_s[r]);
                float xv[8];
                load8(p.v, p.dtype, (size_t)n * kD + 8 * i, xv);
                encode_values(xv, i, p.c.Gv, val_rec(p.c, slot));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Dense rotation for few token-heads (the per-step append of a decode loop): one 256-thread
// block per token-head.  Thread t computes half (t >> 5) & 1 of row 32 (t >> 6) + (t & 31) of
// k' = R k as a binary64 fused chain over 64 columns, and the two halves are added.  Every
// load (the key, the value, the 64 binary16 entries of the row half) is issued at the start,
// so the block costs one round of memory latency plus the 64-step chain.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_append_dense_small(AppendParams p, long N)
{
    __shared__ double kd[kD];
    __shared__ double red[8];
    __shared__ uint32_t rows[4];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const long n = blockIdx.x;
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
#pragma unroll
        for (int q = 0; q < kKeyWords; ++q) kr[q] = rows[q];
        kr[kKeyWords] = norm_corr_word((red[4] + red[5]) + (red[6] + red[7]), (red[0] + red[1]) + (red[2] + red[3]));
    }
    if (t >= 64 && t < 80)
        encode_values(xv, t - 64, p.c.Gv, val_rec(p.c, slot));
}

}  // namespace

hipError_t launch_append(const AppendParams &p, hipStream_t s)
{
    const long N = (long)p.B * p.n_new * p.c.Hkv;
    if (N == 0) return hipSuccess;
    if (p.rot_kind == 1) {
        const long blocks = (N + 15) / 16;
        hipLaunchKernelGGL(k_append_hadamard, dim3((unsigned)blocks), dim3(256), 0, s, p, N);
    } else if (N <= 8192) {
        hipLaunchKernelGGL(k_append_dense_small, dim3((unsigned)N), dim3(256), 0, s, p, N);
    } else {
        const long tiles = (N + 31) / 32;
        const long blocks = tiles < 2048 ? tiles : 2048;
        hipLaunchKernelGGL(k_append_dense, dim3((unsigned)blocks), dim3(128), 0, s, p, N);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Tail of uncompressed recent tokens (lazy updates).  One 256-thread block per sequence,
// so that the block that moves a sequence's tokens also updates its length afterwards.
// A row is one (token, KV head): 128 binary16 = 16 lanes x 16 bytes.
// ---------------------------------------------------------------------------------------
namespace {

__global__ __launch_bounds__(256) void k_tail_append(TailEditParams p)
{
    const int b = blockIdx.x, tid = threadIdx.x;
    const int l0 = p.len[b];
    const int rows = p.n * p.Hkv;
    for (int r = tid >> 4; r < rows; r += 16) {
        const int i = r / p.Hkv, h = r - i * p.Hkv, j = l0 + i;
        if (j >= p.cap) continue;  // past the capacity: dropped
        const int c = tid & 15;    // dims 8c .. 8c + 7
        float x[8];
        const size_t src = (((size_t)b * p.n + i) * p.Hkv + h) * kD + 8 * c;
        const size_t dst = (((size_t)b * p.cap + j) * p.Hkv + h) * kD;
        load8(p.nk, p.dtype, src, x);
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = float_to_half_bits(x[2 * q]) | (float_to_half_bits(x[2 * q + 1]) << 16);
        reinterpret_cast<uint4 *>(p.k + dst)[c] = make_uint4(w[0], w[1], w[2], w[3]);
        load8(p.nv, p.dtype, src, x);
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = float_to_half_bits(x[2 * q]) | (float_to_half_bits(x[2 * q + 1]) << 16);
        reinterpret_cast<uint4 *>(p.v + dst)[c] = make_uint4(w[0], w[1], w[2], w[3]);
        if (p.mass && c == 0) p.mass[((size_t)b * p.cap + j) * p.Hkv + h] = 0.0f;
    }
    __syncthreads();  // every thread has read len[b]
    if (tid == 0) p.len[b] = min(l0 + p.n, p.cap);
}

// Tokens n .. len-1 move to 0 .. len-n-1, in ascending steps of at most n tokens: a step's
// destinations lie below its sources and below every later step's sources, and the barrier
// between steps orders them.
__global__ __launch_bounds__(256) void k_tail_retire(TailEditParams p)
{
    const int b = blockIdx.x, tid = threadIdx.x;
    const int l0 = p.len[b];
    const int n = min(p.n, max(l0, 0));
    const int keep = max(l0, 0) - n;
    const size_t row = (size_t)p.Hkv * kD / 8;  // uint4 per token
    uint4 *k4 = reinterpret_cast<uint4 *>(p.k + (size_t)b * p.cap * p.Hkv * kD);
    uint4 *v4 = reinterpret_cast<uint4 *>(p.v + (size_t)b * p.cap * p.Hkv * kD);
    if (n > 0) {
        for (int j0 = 0; j0 < keep; j0 += n) {
            const int cnt = min(n, keep - j0);
            for (size_t e = tid; e < (size_t)cnt * row; e += 256) {
                const size_t d = (size_t)j0 * row + e;
                k4[d] = k4[d + (size_t)n * row];
                v4[d] = v4[d + (size_t)n * row];
            }
            if (p.mass) {
                float *mb = p.mass + (size_t)b * p.cap * p.Hkv;
                for (int e = tid; e < cnt * p.Hkv; e += 256) mb[j0 * p.Hkv + e] = mb[(j0 + n) * p.Hkv + e];
            }
            __syncthreads();
        }
    }
    __syncthreads();  // every thread has read len[b]
    if (tid == 0) {
        p.len[b] = keep;
        if (p.seq_lens) p.seq_lens[b] += n;
    }
}

// ---------------------------------------------------------------------------------------
// Promotion step of the high-precision tier, one 256-thread block per (KV head, sequence).
// Candidates: the tier's C entries and the n tail tokens just compressed (positions
// seq_lens[b] + j).  Rank = number of candidates ahead (larger mass; equal mass: lower
// position; empty entries last, by index); the C first ranks hold the tier afterwards.
// Leaving entries get their key record's norm/correction word back; entering tokens are
// copied from the tail and their record word is replaced by the marker.  The free-slot list
// and the order of entering tokens are ascending, so the result does not depend on timing.
// ---------------------------------------------------------------------------------------
constexpr uint32_t kHpMarker = 0x7E007E00u;  // binary16 NaN norm and correction
constexpr int kHpMaxCand = 1024;

__device__ __forceinline__ uint32_t *norm_word(const HpUpdateParams &p, int b, int kvh, int pos)
{
    const int page = p.page_table[(size_t)b * p.max_pages + (pos >> p.c.logP)];
    const size_t slot = ((size_t)page * p.c.Hkv + kvh) * p.c.P + (pos & (p.c.P - 1));
    return key_rec(p.c, slot) + kKeyWords;
}

__global__ __launch_bounds__(256) void k_hp_update(HpUpdateParams p)
{
    __shared__ float cm[kHpMaxCand];
    __shared__ int cp[kHpMaxCand];
    __shared__ int rk[kHpMaxCand];
    __shared__ int slot_of_entering[kHpMaxCand];
    const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int Hkv = p.c.Hkv, C = p.hcap, n = p.n, m = C + n;
    const size_t e0 = ((size_t)b * Hkv + kvh) * C;
    const int L0 = p.seq_lens[b];
    constexpr int kEmpty = 0x7FFFFFFF;
    for (int i = tid; i < m; i += 256) {
        if (i < C) {
            const int pos = p.hpos[e0 + i];
            cm[i] = pos >= 0 ? p.hmass[e0 + i] : -INFINITY;
            cp[i] = pos >= 0 ? pos : kEmpty;
        } else {
            const int j = i - C;
            cm[i] = p.tmass[((size_t)b * p.tcap + j) * Hkv + kvh];
            cp[i] = L0 + j;
        }
    }
    __syncthreads();
    for (int i = tid; i < m; i += 256) {
        const float mi = cm[i];
        const int pi = cp[i];
        int r = 0;
#pragma unroll 8
        for (int k = 0; k < m; ++k) {
            const float mk = cm[k];
            const int pk = cp[k];
            r += (mk > mi || (mk == mi && (pk < pi || (pk == pi && k < i)))) ? 1 : 0;
        }
        rk[i] = r;
    }
    __syncthreads();
    // leaving entries: record word restored, entry emptied
    for (int i = tid; i < C; i += 256) {
        if (cp[i] != kEmpty && rk[i] >= C) {
            *norm_word(p, b, kvh, cp[i]) = p.hsaved[e0 + i];
            p.hpos[e0 + i] = -1;
        }
    }
    // free slots (ascending) matched with entering tokens (ascending j), by one thread
    if (tid == 0) {
        int f = 0;
        for (int j = 0; j < n; ++j) {
            if (rk[C + j] < C) {
                while (f < C && cp[f] != kEmpty && rk[f] < C) ++f;  // occupied and staying
                slot_of_entering[j] = f++;
            } else {
                slot_of_entering[j] = -1;
            }
        }
    }
    __syncthreads();
    // entering tokens: 16 threads copy a token's key and value rows, one sets the entry
    for (int r = tid >> 4; r < n; r += 16) {
        const int f = slot_of_entering[r];
        if (f < 0) continue;
        const int c = tid & 15;
        const size_t src = (((size_t)b * p.tcap + r) * Hkv + kvh) * kD;
        const size_t dst = (e0 + f) * kD;
        reinterpret_cast<uint4 *>(p.hk + dst)[c] = reinterpret_cast<const uint4 *>(p.tk + src)[c];
        reinterpret_cast<uint4 *>(p.hv + dst)[c] = reinterpret_cast<const uint4 *>(p.tv + src)[c];
        if (c == 0) {
            const int pos = L0 + r;
            uint32_t *nw = norm_word(p, b, kvh, pos);
            p.hsaved[e0 + f] = *nw;
            *nw = kHpMarker;
            p.hpos[e0 + f] = pos;
            p.hmass[e0 + f] = cm[C + r];
        }
    }
}

}  // namespace

hipError_t launch_hp_update(const HpUpdateParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_hp_update, dim3(p.c.Hkv, p.B), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tail_append(const TailEditParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_tail_append, dim3(p.B), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_tail_retire(const TailEditParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_tail_retire, dim3(p.B), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
