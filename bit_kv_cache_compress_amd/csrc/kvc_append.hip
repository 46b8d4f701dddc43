// Append kernels: encode new keys (sign bits of a random rotation + binary16 norm and
// correction) and values (per-group 4-bit linear codes) into the paged cache.
//
// Method: "H1B-KV" (key design: 1-bit key sketch by random projection, 4-bit linear value
// quantization) with the randomized rotation of "RaBitQCache" (abstract).  The sign of each
// rotated coordinate is the sign of the exact product: for binary16 (and, in practice,
// binary32) inputs every partial sum of R k is exact in binary64.  The randomized Hadamard
// rotation runs its butterflies in binary64; the dense rotation of large appends of binary16
// keys runs on the fp16 matrix cores with a rigorous error bound per coordinate and a
// binary64 sum for the few coordinates inside it (k_append_mfma); the other dense appends
// rotate in binary64 (MFMA f64, or fp64 fma chains for a few keys).
#include "kvc_append_dev.h"

namespace kvc {

namespace {

typedef double double4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Randomized Hadamard rotation (append_hadamard_block): 64 token-heads per 256-thread block.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 4) void k_append_hadamard(AppendParams p, long N)
{
    append_hadamard_block(p, N, blockIdx.x);
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
                if (rb < 2 * p.c.kw) sa += fabs(val);  // dims 16 rb .. 16 rb + 15 of the sketch
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
                    for (int q2 = 0; q2 < p.c.kw; ++q2) kr[q2] = words[v][q2];
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
                if (i == 0) key_rec(p.c, slot)[p.c.kw] = norm_corr_word(ss, sabs_s[r], p.c.sk);
                float xv[8];
                load8(p.v, p.dtype, (size_t)n * kD + 8 * i, xv);
                encode_values(xv, i, p.c.Gv, val_rec(p.c, slot));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Dense rotation on the matrix cores, for binary16 keys without key centers: 16 token-heads
// per wave, k' = R k as v_mfma_f32_16x16x32_f16 with the keys as A (16 tokens x 128 dims) and
// the rotation as B (B[j][o] = R[o][j]).  Binary16 products are exact in binary32, so the only
// error of an output is that of its binary32 sums: at most gamma_128 = 128 u / (1 - 128 u)
// < 7.7e-6 (u = 2^-24) times sum_j |R_oj k_j|, whatever order the matrix core adds in, and by
// Cauchy-Schwarz that sum is at most |R_o| |k| (Euclidean norms: of the row, computed once per
// block in binary64, and of the key, from its binary64 |k|^2).  A coordinate whose |k'_o|
// exceeds 1e-5 |R_o| |k| has the sign of the exact product; the others (rare) take the exact
// sign from a binary64 sum of the 128 products over the wave's lanes.
// The token-heads are taken head by head (n = (b Hkv + h) n_new + t), so that a wave's 16
// records are consecutive slots of a page, written whole.  sum |k'| (for the correction) is
// the binary32 sum of the matrix-core outputs, within 1e-5 relative of the binary64 one.
// ---------------------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBS = kD + 8;  // LDS row stride of the rotation (halves): 16-byte aligned rows

__device__ __forceinline__ half8_t as_half8(uint4 v)
{
    half8_t h;
    __builtin_memcpy(&h, &v, 16);
    return h;
}

// v (64-bit) of lane src
__device__ __forceinline__ size_t from_lane64(size_t v, int src)
{
    const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)v);
    const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)(v >> 32));
    return ((size_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ double xor_lane_d(double v, int m)
{
    const long long x = __double_as_longlong(v);
    const int lo = xor_lane((int)x, m), hi = xor_lane((int)(x >> 32), m);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Input row and slot of token-head n in head-major order.
__device__ __forceinline__ void token_at(const AppendParams &p, uint32_t n, size_t &row, size_t &slot)
{
    const uint32_t nn = (uint32_t)p.n_new, hk = (uint32_t)p.c.Hkv;
    const uint32_t t = n % nn, bh = n / nn;
    const uint32_t h = bh % hk, b = bh / hk;
    row = ((size_t)(b * nn + t) * hk + h) * kD;
    const int pos = p.start_pos[b] + (int)t;
    const int page = p.page_table[(size_t)b * p.max_pages + (pos >> p.c.logP)];
    slot = ((size_t)page * p.c.Hkv + h) * p.c.P + (pos & (p.c.P - 1));
}

__global__ __launch_bounds__(256, 4) void k_append_mfma(AppendParams p, int N)
{
    __shared__ __align__(16) uint16_t Bt[kD * kBS];  // Bt[o][j] = B[j][o]
    __shared__ uint64_t sgn_s[4][32];                // per wave: sign ballots [4 nt + i]
    __shared__ uint64_t unc_s[4][32];                // per wave: uncertain ballots
    __shared__ float sab_s[4][16];                   // per wave: sum |k'| of the tile's tokens
    __shared__ double ss_s[4][16];                   // per wave: |k|^2 of the tile's tokens
    __shared__ float rn_s[kD];                       // |R_o|, rounded up
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int c = tid; c < kD * kD / 8; c += 256) {
        const int o = c >> 4, q = c & 15;  // row o, halves 8 q .. 8 q + 7
        *reinterpret_cast<uint4 *>(&Bt[o * kBS + 8 * q]) = reinterpret_cast<const uint4 *>(p.rot)[c];
    }
    __syncthreads();
    if (tid < kD) {
        double r2 = 0.0;
        for (int j = 0; j < kD; ++j) {
            const double r = (double)half_bits_to_float(Bt[tid * kBS + j]);
            r2 = fma(r, r, r2);
        }
        rn_s[tid] = (float)(sqrt(r2) * (1.0 + 0x1p-20));
    }
    __syncthreads();
    const uint16_t *K = reinterpret_cast<const uint16_t *>(p.k);
    const uint16_t *V = reinterpret_cast<const uint16_t *>(p.v);
    const int m = lane & 15, kb = lane >> 4;  // A layout: token m, dims 8 kb + 32 ks
    const int tv = lane >> 2, jv = lane & 3;  // value layout: token tv, dims 32 jv .. + 31
    float rb[8];  // 1e-5 |R_o| of out dims o = 16 nt + m
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) rb[nt] = 1e-5f * rn_s[16 * nt + m];
    const uint32_t ntiles = ((uint32_t)N + 15u) / 16u;
    for (uint32_t tile = blockIdx.x * 4u + (uint32_t)wave; tile < ntiles; tile += gridDim.x * 4u) {
        const int nvalid = min(16, N - (int)(tile * 16u));
        size_t row = 0, slot = 0;
        if (lane < 16) token_at(p, tile * 16u + (uint32_t)min(lane, nvalid - 1), row, slot);
        const size_t rowA = from_lane64(row, m), rowV = from_lane64(row, tv);
        const size_t slotA = from_lane64(slot, m), slotV = from_lane64(slot, tv);
        uint4 a[4], vr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const uint4 *>(K + rowA + 32 * ks + 8 * kb);
#pragma unroll
        for (int q = 0; q < 4; ++q) vr[q] = *reinterpret_cast<const uint4 *>(V + rowV + 32 * jv + 8 * q);
        if (p.c.kf16 && m < nvalid) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<uint4 *>(p.c.kf16 + slotA * kD + 32 * ks + 8 * kb) = a[ks];
        }
        // |k|^2 (binary64) of token m: this lane's 32 dims, then lanes m, m + 16, m + 32, m + 48
        double ss = 0.0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t w[4] = {a[ks].x, a[ks].y, a[ks].z, a[ks].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = half_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                ss = fma((double)x, (double)x, ss);
            }
        }
        ss += xor_lane_d(ss, 16);
        ss += xor_lane_d(ss, 32);
        if (kb == 0) ss_s[wave][m] = ss;
        // |k| of tokens 4 kb + i (the bound's key factor), from lanes 4 kb + i
        float kn[4];
        {
            const float knm = sqrtf((float)ss);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kn[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * kb + i) << 2, __float_as_int(knm)));
        }
        // the products: acc[nt] holds out dim 16 nt + m of tokens 4 kb + i in element i
        f32x4_t acc[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[nt] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            uint4 bw[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                bw[ks] = *reinterpret_cast<const uint4 *>(&Bt[(16 * nt + m) * kBS + 32 * ks + 8 * kb]);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a[ks]), as_half8(bw[ks]), acc[nt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);  // one output tile's operands at a time
        }
        // signs, certified against the bound; sum |k'| over the sketch's dims
        // the 32 sign ballots (and, when some coordinate is uncertain, the 32 uncertainty
        // ballots) go to LDS from lanes 0..31, ballot k = 4 nt + i in lane k
        uint64_t any = 0;
        float sa[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        int sg_lo = 0, sg_hi = 0, un_lo = 0, un_hi = 0;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = acc[nt][i];
                const float b = rb[nt] * kn[i];  // >= 1e-5 sum_j |R_oj k_j|
                const uint64_t sg = __builtin_amdgcn_ballot_w64(!(v < 0.0f));
                const uint64_t un = __builtin_amdgcn_ballot_w64(!(fabsf(v) > b));
                const bool mine = lane == 4 * nt + i;
                sg_lo = mine ? (int)(uint32_t)sg : sg_lo;
                sg_hi = mine ? (int)(uint32_t)(sg >> 32) : sg_hi;
                un_lo = mine ? (int)(uint32_t)un : un_lo;
                un_hi = mine ? (int)(uint32_t)(un >> 32) : un_hi;
                any |= un;
                if (nt < 2 * p.c.kw) sa[i] += fabsf(v);
            }
        }
        if (lane < 32) {
            sgn_s[wave][lane] = ((uint64_t)(uint32_t)sg_hi << 32) | (uint32_t)sg_lo;
            if (any) unc_s[wave][lane] = ((uint64_t)(uint32_t)un_hi << 32) | (uint32_t)un_lo;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) sa[i] += xor_lane(sa[i], o);
            if (m == 0) sab_s[wave][4 * kb + i] = sa[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (any) {
            // exact signs of the uncertain coordinates: lane l adds the products of dims
            // 2 l, 2 l + 1 in binary64 (exact for binary16 operands), summed over the wave
            for (int k = 0; k < 32; ++k) {
                uint64_t u = unc_s[wave][k];
                const int nt = k >> 2, i = k & 3;
                while (u) {
                    const int bit = __builtin_ctzll(u);
                    u &= u - 1;
                    const int tok = 4 * (bit >> 4) + i, o = 16 * nt + (bit & 15);
                    const size_t r = from_lane64(row, tok);
                    const uint32_t xw = *reinterpret_cast<const uint32_t *>(K + r + 2 * lane);
                    const uint32_t bw = *reinterpret_cast<const uint32_t *>(&Bt[o * kBS + 2 * lane]);
                    double s = (double)half_bits_to_float(xw & 0xFFFFu) * (double)half_bits_to_float(bw & 0xFFFFu);
                    s += (double)half_bits_to_float(xw >> 16) * (double)half_bits_to_float(bw >> 16);
#pragma unroll
                    for (int q = 32; q > 0; q >>= 1) s += xor_lane_d(s, q);
                    if (lane == 0) {
                        const uint64_t b1 = 1ull << bit;
                        sgn_s[wave][k] = (s < 0.0) ? (sgn_s[wave][k] & ~b1) : (sgn_s[wave][k] | b1);
                    }
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // key record of token tv: word jv (dims 32 jv .. 32 jv + 31: out tiles 2 jv, 2 jv + 1),
        // and the norm/correction word
        if (tv < nvalid) {
            const int g = tv >> 2, i = tv & 3;
            const uint32_t lo = (uint32_t)(sgn_s[wave][4 * (2 * jv) + i] >> (16 * g)) & 0xFFFFu;
            const uint32_t hi = (uint32_t)(sgn_s[wave][4 * (2 * jv + 1) + i] >> (16 * g)) & 0xFFFFu;
            uint32_t *kr = key_rec(p.c, slotV);
            if (jv < p.c.kw) kr[jv] = lo | (hi << 16);
            if (jv == 0) {
                const double sabs = (double)sab_s[wave][tv];
                kr[p.c.kw] = norm_corr_word(ss_s[wave][tv], sabs, p.c.sk);
            }
            float x[32];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w[4] = {vr[q].x, vr[q].y, vr[q].z, vr[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[8 * q + 2 * e] = half_bits_to_float(w[e] & 0xFFFFu);
                    x[8 * q + 2 * e + 1] = half_bits_to_float(w[e] >> 16);
                }
            }
            encode_values32(x, jv, p.c.Gv, val_rec(p.c, slotV));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the LDS slices are rewritten
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ---------------------------------------------------------------------------------------
// Dense rotation for few token-heads (append_small_block): one 256-thread block per
// token-head.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_append_dense_small(AppendParams p, long N)
{
    append_small_block(p, N, blockIdx.x);
}

}  // namespace

long fused_append_blocks(const AppendParams &p)
{
    const long N = (long)p.B * p.n_new * p.c.Hkv;
    if (N == 0) return 0;
    if (p.rot_kind == 1) return (N + 63) / 64;
    return N <= 8192 ? N : 0;
}

hipError_t launch_append(const AppendParams &p, hipStream_t s)
{
    const long N = (long)p.B * p.n_new * p.c.Hkv;
    if (N == 0) return hipSuccess;
    // dense rotation, binary16 keys without centers: the rotation on the matrix cores (16
    // token-heads per wave); the randomized Hadamard rotation's butterflies cost less than its
    // 128 x 128 product
    const bool mfma = p.rot_kind == 0 && p.dtype == 0 && !p.c.kc && N > 8192 && N < (1L << 31);
    if (mfma) {
        const long mblocks = ((N + 15) / 16 + 3) / 4;
        const unsigned blocks = (unsigned)(mblocks < 1024 ? mblocks : 1024);
        KVC_LAUNCH(k_append_mfma, dim3(blocks), dim3(256), s, p, (int)N);
    } else if (p.rot_kind == 1) {
        const long blocks = (N + 63) / 64;
        KVC_LAUNCH(k_append_hadamard, dim3((unsigned)blocks), dim3(256), s, p, N);
    } else if (N <= 8192) {
        KVC_LAUNCH(k_append_dense_small, dim3((unsigned)N), dim3(256), s, p, N);
    } else {
        const long tiles = (N + 31) / 32;
        const long blocks = tiles < 2048 ? tiles : 2048;
        KVC_LAUNCH(k_append_dense, dim3((unsigned)blocks), dim3(128), s, p, N);
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
    return key_rec(p.c, slot) + p.c.kw;
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
    KVC_LAUNCH(k_hp_update, dim3(p.c.Hkv, p.B), dim3(256), s, p);
    return hipGetLastError();
}

hipError_t launch_tail_append(const TailEditParams &p, hipStream_t s)
{
    KVC_LAUNCH(k_tail_append, dim3(p.B), dim3(256), s, p);
    return hipGetLastError();
}

hipError_t launch_tail_retire(const TailEditParams &p, hipStream_t s)
{
    KVC_LAUNCH(k_tail_retire, dim3(p.B), dim3(256), s, p);
    return hipGetLastError();
}

}  // namespace kvc
