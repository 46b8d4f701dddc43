// Decode kernels: query preparation, binary x INT4 proxy scores, adaptive Top-p (bin
// distances, histogram and threshold, ordered selection), chunked attention over the 4-bit
// values, and the split-K merge.
//
// Method: "RaBitQCache" (abstract and key design: int4 query, binary x INT4 proxy score,
// adaptive Top-p) and "H1B-KV" (technical framework: attention weights from the 1-bit key
// sketch, output from the 4-bit values).
//
// Work decomposition.  A sequence is cut into chunks of CH tokens (CH a power of two,
// 256..8192).  One 256-thread block works on one (chunk, KV head, sequence) and on GB <= 4
// of the query heads that share the KV head (GQA), so every key word and value byte it
// streams from HBM serves all GB heads.  The page ids of a chunk are read once into LDS, and
// each thread issues all of its loads of a pass before using any of them, so that a block
// keeps several KB of HBM reads in flight.  Partial results (max score, weight sum, weighted
// value sum) of all chunks are merged per (sequence, query head) at the end.
#include <mutex>

#include "kvc_append_dev.h"
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

thread_local StageTiming g_stage_timing = {nullptr, nullptr};

// Result words of the argument checker (k_check), one copy per device.
__device__ int32_t g_check_flag[4];

// Workspace of kv_decode_attend_noalloc: every device the library runs on holds its own copy
// until the process ends.  Host code reaches it only through the per-device address that
// static_scratch() takes with hipGetSymbolAddress (the array's name in host code is a
// host-side stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// First query head of block (hb = kv head * nsub + sub) and its KV head.
__device__ __forceinline__ void block_heads(const DecodeGeom &g, int hb, int &kvh, int &hq0)
{
    kvh = hb / g.nsub;
    const int sub = hb - kvh * g.nsub;
    hq0 = kvh * g.G + sub * g.GB;
}

__device__ __forceinline__ size_t chunk_slot(const CacheView &c, const int *pages, int p0, int kvh, int t)
{
    return ((size_t)pages[(t >> c.logP) - p0] * c.Hkv + kvh) * c.P + (t & (c.P - 1));
}

// Key record of a slot: the sign bytes (one 16- or 8-byte load at 4-byte alignment; a
// 64-bit sketch leaves the upper two words zero) and the norm/corr word.
__device__ __forceinline__ void load_key(const CacheView &c, size_t slot, uint4 &kb, uint32_t &nc)
{
    const uint32_t *kr = key_rec(c, slot);
    if (c.kw == 4) {
        __builtin_memcpy(&kb, kr, 16);
    } else {
        uint2 lo;
        __builtin_memcpy(&lo, kr, 8);
        kb = make_uint4(lo.x, lo.y, 0u, 0u);
    }
    nc = kr[c.kw];
}

// load_key for a record width known at compile time (KW sign words): the fast paths are
// instantiated per width, so their unrolled key loads carry no width test.
template <int KW>
__device__ __forceinline__ void load_key_t(const CacheView &c, size_t slot, uint4 &kb, uint32_t &nc)
{
    const uint32_t *kr = c.keys + slot * (KW + 1);
    if constexpr (KW == 4) {
        __builtin_memcpy(&kb, kr, 16);
    } else {
        uint2 lo;
        __builtin_memcpy(&lo, kr, 8);
        kb = make_uint4(lo.x, lo.y, 0u, 0u);
    }
    nc = kr[KW];
}

// Block-wide reduction of GB values per thread (256 threads); result broadcast in LDS.
template <int GB, typename T, typename Op>
__device__ __forceinline__ void block_reduce(T (&v)[GB], T *red /* [4][GB] */, T *out /* [GB] */, Op op)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        T x = v[h];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) x = op(x, __shfl_xor(x, o));
        if (lane == 0) red[wave * GB + h] = x;
    }
    __syncthreads();
    if (threadIdx.x < GB) {
        T x = red[threadIdx.x];
        for (int w = 1; w < 4; ++w) x = op(x, red[w * GB + threadIdx.x]);
        out[threadIdx.x] = x;
    }
    __syncthreads();
}

struct MaxI { __device__ int operator()(int a, int b) const { return a > b ? a : b; } };
struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct SumF { __device__ float operator()(float a, float b) const { return a + b; } };
struct SumI { __device__ int operator()(int a, int b) const { return a + b; } };

// ---------------------------------------------------------------------------------------
// Exact attention over the binary16 tail (lazy updates) for query head h of sequence b, by
// a 256-thread block.  The tail tokens and then the entries of the high-precision tier (KV
// head of h; empty entries with weight 0) form one index space.  A pass covers 256 of them:
// thread t scores token t (<q, k> as a binary32 fma chain over the 128 dims) while thread
// (dg, ts) = (t mod 16, t / 16) already holds the values of dims 8 dg .. 8 dg + 7 of tokens
// ts + 16 i, i < 16, so that every load of the pass is in flight at once.  The block takes
// the max and the weights exp2((s - m) log2e / sqrt(D)) with a running max over passes;
// thread (dg, ts) sums its 16 weighted values, and the 16 token slices are added at the end.  With key centers the scores are <q, k> - <q, c> (the frame of the
// centered proxy scores).  Writes the partial
// (m, l, o[128]) that the merge adds to the chunk partials (m = -inf and zeros for an
// empty tail).
// ---------------------------------------------------------------------------------------
// Exact score <q, k> of one binary16 key against the binary32 query in LDS: a binary32 fma
// chain over the 128 dims (dim 0 first).
__device__ __forceinline__ float exact_dot(const uint16_t *k, const float *qs)
{
    const uint4 *kr = reinterpret_cast<const uint4 *>(k);
    uint4 kk[kD / 8];
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) kk[c] = kr[c];
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
        const uint32_t w[4] = {kk[c].x, kk[c].y, kk[c].z, kk[c].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qs[8 * c + e], half_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), a);
    }
    return a;
}

// <q, c> of the KV head's key center, by the first two waves of the block (q in qs); every
// thread of the block gets the sum.  red2 is two floats of LDS.
__device__ __forceinline__ float center_dot(const float *center, int kvh, const float *qs, float *red2)
{
    const int tid = threadIdx.x;
    const float x = tid < kD ? qs[tid] * center[(size_t)kvh * kD + tid] : 0.0f;
    const float cs = wave_sum(x);
    if (tid == 0 || tid == 64) red2[tid >> 6] = cs;
    __syncthreads();
    const float qc = red2[0] + red2[1];
    __syncthreads();  // red2 may be reused
    return qc;
}

__device__ __forceinline__ void tail_attend(const TailParams &p, int bh)
{
    constexpr int T = 256, NS = T / 16, NV = T / NS;  // tokens per pass, token slices, values per thread
    constexpr int NW = T / 64;
    __shared__ float qs[kD];
    __shared__ float ws[T];
    __shared__ float part[NS][kD];
    __shared__ float red[2][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = bh / p.Hq, h = bh - b * p.Hq, kvh = h / p.G;
    if (tid < kD) qs[tid] = p.q[(size_t)bh * kD + tid];
    __syncthreads();
    // centered cache: exact scores move to the same frame, <q, k> - <q, c>
    const float qc = p.center ? center_dot(p.center, kvh, qs, red[0]) : 0.0f;
    const int dg = tid & 15, ts = tid >> 4;
    // one index space: tail tokens 0 .. nt-1, then the tier entries of this KV head
    const int nt = p.k ? min(max(p.len[b], 0), p.cap) : 0;
    const int nh = p.hk ? p.hcap : 0;
    const int ntot = nt + nh;
    const size_t trow = (size_t)p.Hkv * kD;
    const uint16_t *tk = p.k ? p.k + ((size_t)b * p.cap * p.Hkv + kvh) * kD : nullptr;
    const uint16_t *tv = p.v ? p.v + ((size_t)b * p.cap * p.Hkv + kvh) * kD : nullptr;
    const size_t e0 = ((size_t)b * p.Hkv + kvh) * p.hcap;
    const uint16_t *hk = p.hk ? p.hk + e0 * kD : nullptr;
    const uint16_t *hv = p.hv ? p.hv + e0 * kD : nullptr;
    float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    for (int t0 = 0; t0 < ntot; t0 += T) {
        uint4 vr[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int u = t0 + ts + NS * i;
            const uint16_t *vp = u < nt ? tv + u * trow : hv + (size_t)(u - nt) * kD;
            vr[i] = u < ntot ? *reinterpret_cast<const uint4 *>(vp + 8 * dg) : make_uint4(0u, 0u, 0u, 0u);
        }
        const int u = t0 + tid;
        // empty tier entries are read like the others (the arrays are whole) and masked after,
        // so that the key loads do not wait for the position load
        float s = -INFINITY;
        if (u < ntot) s = exact_dot(u < nt ? tk + u * trow : hk + (size_t)(u - nt) * kD, qs) - qc;
        if (u >= nt && (u >= ntot || p.hpos[e0 + (u - nt)] < 0)) s = -INFINITY;
        const float wm = wave_max(s);
        if (lane == 0) red[0][wave] = wm;
        __syncthreads();
        float mnew = m;
#pragma unroll
        for (int w = 0; w < NW; ++w) mnew = fmaxf(mnew, red[0][w]);
        const float scale = (m == -INFINITY) ? 0.0f : exp2f((m - mnew) * p.klog);
        const float w = (s == -INFINITY) ? 0.0f : exp2f((s - mnew) * p.klog);
        ws[tid] = w;
        const float wsum = wave_sum(w);
        if (lane == 0) red[1][wave] = wsum;
        __syncthreads();
        float lsum = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) lsum += red[1][w2];
        l = l * scale + lsum;
        m = mnew;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= scale;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float wi = ws[ts + NS * i];
            const uint32_t keep = wi != 0.0f ? 0xFFFFFFFFu : 0u;  // empty entries hold anything
            const uint32_t x[4] = {vr[i].x & keep, vr[i].y & keep, vr[i].z & keep, vr[i].w & keep};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = fmaf(wi, half_bits_to_float((x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), o[e]);
        }
        __syncthreads();  // ws and red are rewritten by the next pass
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[ts][8 * dg + e] = o[e];
    __syncthreads();
    if (tid < kD) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NS; ++j) acc += part[j][tid];
        p.to[(size_t)bh * kD + tid] = acc;
    }
    if (tid == 0) {
        p.tm[bh] = m;
        p.tl[bh] = l;
    }
}

// ---------------------------------------------------------------------------------------
// Query preparation (one block per (sequence, query head), one thread per dim; with a tail,
// blocks BH .. 2 BH - 1 run the tail attention of the same heads alongside, and the blocks
// after those encode the new tokens of a fused append; with either, all blocks have 256
// threads, of which the query preparation uses the first 128):
//   dense:    q'_r = fmaf chain over j ascending of R[r][j] * q_j (binary32)
//   hadamard: x = sigma * q, in-place fast Walsh-Hadamard butterflies h = 1..64 (binary32),
//             q' = x * fp32(1/sqrt(D))
//   over the sketch's dims r < sk (the others get code 0):
//   v_l = min q', delta = (max q' - v_l) / 15, u = clamp(rint((q' - v_l) / delta), 0, 15)
//   (u = 0 when delta == 0), or clamp(floor((q' - v_l) / delta + U), 0, 15) with the
//   caller's uniform U under stochastic rounding; the codes in dot8 order; c0 = v_l/sqrt(sk),
//   c1 = delta/sqrt(sk).
// ---------------------------------------------------------------------------------------
// EXTRA: the blocks the launch carries past the query heads' -- 0 none, 1 the binary16 tail
// and any appends, 2 randomized-Hadamard appends only, 3 dense appends only -- so that a
// launch compiles in (and holds registers for) only the paths it runs.
template <int EXTRA>
__global__ __launch_bounds__(256) void k_qprep(QprepParams p, float isd)
{
    __shared__ float xs[kD];
    __shared__ int us[kD];
    __shared__ float redf[4];
    __shared__ int redi[4];
    if (EXTRA != 0 && (int)blockIdx.x >= p.BH) {
        const long tb = p.has_tail ? p.BH : 0;  // tail blocks
        const long ab = (long)blockIdx.x - p.BH - tb;
        if constexpr (EXTRA == 1) {
            if (ab < 0) {
                tail_attend(p.tail, (int)blockIdx.x - p.BH);
            } else if (p.app.rot_kind == 1) {
                append_hadamard_block(p.app, p.app_N, ab);
            } else {
                append_small_block(p.app, p.app_N, ab);
            }
        } else if constexpr (EXTRA == 2) {
            append_hadamard_block(p.app, p.app_N, ab);
        } else if constexpr (EXTRA == 3) {
            append_small_block(p.app, p.app_N, ab);
        }
        return;
    }
    if (threadIdx.x >= kD) return;  // whole waves: blocks of 256 threads when a tail runs alongside
    const int bh = blockIdx.x, r = threadIdx.x;
    if (p.order_ctr && (bh | r) == 0) {  // the dispatch slots of the threshold pass, two kernels on
        p.order_ctr[0] = 0;
        p.order_ctr[1] = 0;
    }
    const int lane = r & 63, wave = r >> 6;
    const float *q = p.q + (size_t)bh * kD;
    float x;
    if (p.rot_kind == 0) {
        const uint4 *Rr = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.rot) + r * kD);
        uint4 row[kD / 8];
#pragma unroll
        for (int c = 0; c < kD / 8; ++c) row[c] = Rr[c];
        xs[r] = q[r];
        __syncthreads();
        float a = 0.0f;
#pragma unroll
        for (int c = 0; c < kD / 8; ++c) {
            const uint32_t w[4] = {row[c].x, row[c].y, row[c].z, row[c].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 8 * c + e;
                const float rj = half_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                a = (j == 0) ? rj * xs[0] : fmaf(rj, xs[j], a);
            }
        }
        x = a;
    } else {
        const uint32_t *sg = reinterpret_cast<const uint32_t *>(p.rot);
        float v = q[r];
        if ((sg[r >> 5] >> (r & 31)) & 1u) v = -v;
        xs[r] = v;
        for (int h = 1; h < kD; h <<= 1) {
            __syncthreads();
            const float a = xs[r & ~h], b = xs[r | h];
            const float nv = (r & h) ? (a - b) : (a + b);
            __syncthreads();
            xs[r] = nv;
        }
        __syncthreads();
        x = xs[r] * isd;
    }
    // the range of the sketch's dims (the first sk rotated coordinates)
    float mn = r < p.sk ? x : INFINITY, mx = r < p.sk ? x : -INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    if (lane == 0) {
        redf[wave] = mn;
        redf[2 + wave] = mx;
    }
    __syncthreads();
    const float vl = fminf(redf[0], redf[1]);
    const float vr = fmaxf(redf[2], redf[3]);
    const float delta = (vr - vl) / 15.0f;
    int u = 0;
    if (delta != 0.0f && r < p.sk) {  // dims past the sketch keep code 0
        const float tq = (x - vl) / delta;
        float t = p.dither ? floorf(tq + p.dither[(size_t)bh * kD + r]) : rintf(tq);
        t = fminf(fmaxf(t, 0.0f), 15.0f);
        u = (int)t;
    }
    int su = wave_sum_i(u);
    int s3 = wave_sum_i((r & 3) == 3 ? u : 0);  // the codes of dims 3 mod 4 (k_score_topp_mf)
    if (lane == 0) {
        redi[wave] = su;
        redi[2 + wave] = s3;
    }
    __syncthreads();  // everyone has read xs
    us[r] = u;
    __syncthreads();
    if (r < 16) {
        // word 4w + k: nibble m holds the code of dim 32w + 4m + k
        const int w = r >> 2, k = r & 3;
        uint32_t word = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m) word |= (uint32_t)us[32 * w + 4 * m + k] << (4 * m);
        p.qnib[(size_t)bh * 16 + r] = word;
    }
    {
        // the codes as the fp8 A operand of k_score_topp_mf, byte r = 32 group + index: it
        // meets K = 16 group + index (index < 16) or 64 + 16 group + index - 16 of the fp4 key
        // operand, where K = 32 j + 8 v + m carries bit 4m + v of key word j as 1/2, 1, 2 times
        // the bit for v = 0..2 (the code is scaled by 4, 2, 1 to match) and as 1 - 2 bit for
        // v = 3 (the code is negated)
        const int ga = r >> 5, pa = r & 31;
        const int K = pa < 16 ? 16 * ga + pa : 64 + 16 * ga + (pa - 16);
        const int j = K >> 5, v = (K >> 3) & 3, m = K & 7;
        const int uc = us[32 * j + 4 * m + v];
        const uint32_t f8 = fp8_e4m3_small(uc << (v == 0 ? 2 : v == 1 ? 1 : 0));
        p.qa[(size_t)bh * kD + r] = (uint8_t)(v == 3 && uc ? f8 | 0x80u : f8);  // -u for v = 3
    }
    su = redi[0] + redi[1];
    s3 = redi[2] + redi[3];
    // (c0, c1, sumu as integer bits, s3 - sumu as a float: the matrix-core products' offset)
    if (r == 0) p.qpar[bh] = make_float4(vl * p.isk, delta * p.isk, __int_as_float(su), (float)(s3 - su));
    if (p.dbg_codes) p.dbg_codes[(size_t)bh * kD + r] = (uint8_t)u;
    if (r == 0 && p.dbg_params) {
        p.dbg_params[bh * 4 + 0] = vl;
        p.dbg_params[bh * 4 + 1] = delta;
        p.dbg_params[bh * 4 + 2] = vl * p.isk;
        p.dbg_params[bh * 4 + 3] = delta * p.isk;
    }
    if (r == 0 && p.dbg_sumu) p.dbg_sumu[bh] = su;
}

// ---------------------------------------------------------------------------------------
// Score pass (Top-p first pass, and debug scores): one wave per (chunk, KV head, sequence)
// computes the proxy score of every token of the chunk for GB query heads.  Writes the bin
// distance to the chunk's top bin (uint16, saturated at 8192: no token that far below a
// chunk's top can be selected, since the threshold distance is < 8192) and the chunk's top
// bin.  Lane l scores tokens l, l + 64, ... (coalesced 16-byte key loads, 8 in flight), then
// stores the distances of 8 consecutive tokens per 16-byte store.  One-wave blocks need no
// block barrier, so the load, compute and store phases of different waves overlap freely.
// ---------------------------------------------------------------------------------------
template <int GB, bool DEBUG, int CHMAX>
__global__ __launch_bounds__(64) void k_score(ScoreParams p)
{
    __shared__ int ebuf[GB * CHMAX];
    __shared__ int pages[CHMAX / 16 + 1];
    __shared__ uint32_t qsh[GB * 16];
    __shared__ float4 qps[GB];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int lane = threadIdx.x;
    const int bh0 = b * g.Hq + hq0;
    if (lane < GB * 16) qsh[lane] = p.qnib[(size_t)(bh0 + lane / 16) * 16 + (lane & 15)];
    if (lane < GB) qps[lane] = p.qpar[bh0 + lane];
    const int p0 = t0 >> p.c.logP;
    const int np = ((t0 + n - 1) >> p.c.logP) - p0 + 1;
    for (int i = lane; i < np; i += 64) pages[i] = g.page_table[(size_t)b * g.max_pages + p0 + i];
    __syncthreads();
    QueryState<GB> qs;
    read_query<GB>(qs, qsh, qps);
    int lm[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) lm[h] = -kBinClamp;
    for (int k0 = 0; k0 < n; k0 += 8 * 64) {
        uint4 kb[8];
        uint32_t nc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tl = k0 + lane + 64 * u;
            if (tl < n) {
                load_key(p.c, chunk_slot(p.c, pages, p0, kvh, t0 + tl), kb[u], nc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tl = k0 + lane + 64 * u;
            if (tl < n) {
                float s[GB];
                int A[GB];
                score_key<GB>(kb[u], nc[u], qs, s, A, p.c.sk);
#pragma unroll
                for (int h = 0; h < GB; ++h) {
                    const int e = score_bin(s[h], p.kbin);
                    ebuf[h * CHMAX + tl] = e;
                    lm[h] = max(lm[h], e);
                    if (DEBUG) {
                        if (p.dbg_scores) p.dbg_scores[(size_t)(bh0 + h) * g.ld + t0 + tl] = s[h];
                        if (p.dbg_iscores) p.dbg_iscores[(size_t)(bh0 + h) * g.ld + t0 + tl] = A[h];
                    }
                }
            }
        }
    }
    if (!p.dl) return;
#pragma unroll
    for (int h = 0; h < GB; ++h) lm[h] = wave_max_i(lm[h]);
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GB; ++h) p.lmax[(size_t)(bh0 + h) * g.NC + chunk] = lm[h];
    }
    __syncthreads();  // ebuf written by other lanes
    for (int base = 8 * lane; base < n; base += 8 * 64) {
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int a = base + 2 * q, c = a + 1;
                const uint32_t da = a < n ? (uint32_t)min(lm[h] - ebuf[h * CHMAX + a], kBins) : kBins;
                const uint32_t dc = c < n ? (uint32_t)min(lm[h] - ebuf[h * CHMAX + c], kBins) : kBins;
                w[q] = da | (dc << 16);
            }
            *reinterpret_cast<uint4 *>(p.dl + (size_t)(bh0 + h) * g.Lpad + t0 + base) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Top-p score pass (no debug output): one wave per 512-token chunk, KV head and sequence.
// Lane l scores tokens l + 64 u (u < 8; 16-byte key loads coalesce over the wave).  Page ids
// are turned into 32-bit slot bases in LDS once, so a token's slot is one LDS read and an
// add.  There is no per-token branch: past the sequence end a lane re-reads the last token
// and its bin is forced below every real one.  The bins stay in registers; after the wave
// max, each lane stores its tokens' 16-bit distances (128-byte coalesced stores), and every
// position of the chunk is written (kBins past the end).
// ---------------------------------------------------------------------------------------
// At most 128 VGPRs (4 waves per SIMD requested); the compiler then fits the kernel in 70,
// 7 waves per SIMD, which the key-load latency needs.
template <int GB, int KW>
__global__ __launch_bounds__(64, 4) void k_score_topp(ScoreParams p)
{
    constexpr int CH = kTopPChunk;
    constexpr int U = CH / 64;  // tokens per lane
    constexpr int kNone = -2 * kBinClamp;
    __shared__ uint32_t pbase[CH / 16 + 1];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * CH;
    if (t0 >= L) return;
    const int n = min(CH, L - t0);
    const int lane = threadIdx.x;
    const int bh0 = b * g.Hq + hq0;
    const int logP = p.c.logP;
    const int p0 = t0 >> logP;
    const int np = ((t0 + n - 1) >> logP) - p0 + 1;
    for (int i = lane; i < np; i += 64)
        pbase[i] = ((uint32_t)g.page_table[(size_t)b * g.max_pages + p0 + i] * (uint32_t)p.c.Hkv + (uint32_t)kvh)
                   << logP;
    __syncthreads();
    // the query state is wave-uniform: scalar loads keep it in SGPRs, which the dot8
    // instructions read directly
    QueryState<GB> qs;
#pragma unroll
    for (int h = 0; h < GB; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) qs.nib[h][i] = p.qnib[(size_t)(bh0 + h) * 16 + i];
        const float4 pq = p.qpar[bh0 + h];
        qs.c0[h] = pq.x;
        qs.c1[h] = pq.y;
        qs.sumu[h] = __float_as_int(pq.z);
    }
    uint32_t slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + min(lane + 64 * u, n - 1);
        slot[u] = pbase[(t >> logP) - p0] + (uint32_t)(t & ((1 << logP) - 1));
    }
    int e[U][GB];
    int lm[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) lm[h] = kNone;
    // every key load of the chunk is issued before any arithmetic (the scheduling barrier
    // keeps the compiler from sinking loads next to their uses, which would serialize the
    // round trips)
    uint4 kb[U];
    uint32_t nc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        load_key_t<KW>(p.c, slot[u], kb[u], nc[u]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float s[GB];
        int A[GB];
        score_key<GB>(kb[u], nc[u], qs, s, A, 32 * KW);
        // min() rather than a select, so that the score is computed on every lane
        // instead of behind a branch
        const int lim = lane + 64 * u < n ? INT_MAX : kNone;
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const int ev = min(score_bin(s[h], p.kbin), lim);
            e[u][h] = ev;
            lm[h] = max(lm[h], ev);
        }
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) lm[h] = wave_max_i(lm[h]);
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GB; ++h) p.lmax[(size_t)(bh0 + h) * g.NC + chunk] = lm[h];
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        uint16_t *row = p.dl + (size_t)(bh0 + h) * g.Lpad + t0 + lane;
#pragma unroll
        for (int u = 0; u < U; ++u) row[64 * u] = (uint16_t)min(lm[h] - e[u][h], kBins);
    }
}

// ---------------------------------------------------------------------------------------
// Top-p score pass on the matrix cores, for blocks of 4 query heads (GQA groups of 4 or
// more).  Same work split, loads and outputs as k_score_topp; the binary x INT4 products
// run as v_mfma_scale_f32_16x16x128_f8f6f4 with the query codes as the fp8 (e4m3) A
// operand and the key sign bits as the fp4 (e2m1) B operand (16 columns: tokens), four
// tiles of 16 tokens per 64-token group:
//  - lane l holds token 64u + l of group u.  A 4 x 4 block transpose of its four key words
//    over the 16-lane rows (two permlane32 and two permlane16 swaps) leaves, in register t,
//    word j of token 64u + 16t + n in lane 16j + n: the B operand of tile t.
//  - bit 4m + v of a word goes to nibble m of B register v, as 0x1 (0.5), 0x2 (1), 0x4 (2)
//    for v = 0, 1, 2, with the query codes scaled by 4, 2, 1: each product is 2 * bit * u.
//    For v = 3 the bit stays in place, as the sign of the nibble 0x2 (+1 or -1 for a clear
//    or set bit: one and-or), against the code -u: the product is 2 * bit * u - u, and the
//    sum of those u (the codes of dims 3 mod 4) is added back through the accumulator.
//  - the A operand of tile t holds head h in row 4t + h and zeros in the other rows, and
//    the four tiles accumulate into one result, which starts at -sumu of head h in
//    register h (plus the dims 3 mod 4 sum).  Rows 4t' .. 4t' + 3 of the result (registers 0..3 of lanes 16t' + n)
//    then hold A of the 4 heads for token 64u + 16t' + n: lane l ends with its own token.
// Products and sums are integers below 2^12, exact in binary32: A = 2 ip - sumu and the
// score are bit-identical to the dot8 form.
// ---------------------------------------------------------------------------------------
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

// (a & m) | c in one instruction (VOP3 takes no literal here, and the compiler splits the
// two-constant form in two): m from a scalar register, c from a vector register
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);  // a.hi <-> b.lo
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);  // odd rows of a <-> even rows of b
    a = r[0];
    b = r[1];
}

// The binary x INT4 products of this lane's key with 4 query heads on the matrix cores (the
// transpose, operands and tiles described above): register h of the result is
// A = 2 sum_r bit_r u_r - sumu of head h for the lane's own token.  qa(t) gives the A
// operand of tile t; msu holds the accumulator start of each head.
template <typename QA>
__device__ __forceinline__ v4f_t key_products4(const uint4 &kb, const v4f_t &msu, QA qa)
{
    uint32_t w[4] = {kb.x, kb.y, kb.z, kb.w};
    swap32(w[0], w[2]);
    swap32(w[1], w[3]);
    swap16(w[0], w[1]);
    swap16(w[2], w[3]);
    const uint32_t plus1 = 0x22222222u;  // every nibble +1 (fp4 e2m1 0x2)
    v4f_t d = msu;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const v8i_t bt = {(int)(w[t] & 0x11111111u), (int)(w[t] & 0x22222222u), (int)(w[t] & 0x44444444u),
                          (int)and_or(w[t], 0x88888888u, plus1), 0, 0, 0, 0};
        d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa(t), bt, d, 0, 4, 0, 127, 0, 127);
    }
    return d;
}

template <int KW>
__global__ __launch_bounds__(64, 4) void k_score_topp_mf(ScoreParams p)
{
    constexpr int GB = 4;
    constexpr int CH = kTopPChunk;
    constexpr int U = CH / 64;  // 64-token groups
    constexpr int kNone = -2 * kBinClamp;
    __shared__ uint32_t pbase[CH / 16 + 1];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * CH;
    if (t0 >= L) return;
    const int n = min(CH, L - t0);
    const int lane = threadIdx.x;
    const int bh0 = b * g.Hq + hq0;
    const int logP = p.c.logP;
    const int p0 = t0 >> logP;
    const int np = ((t0 + n - 1) >> logP) - p0 + 1;
    for (int i = lane; i < np; i += 64)
        pbase[i] = ((uint32_t)g.page_table[(size_t)b * g.max_pages + p0 + i] * (uint32_t)p.c.Hkv + (uint32_t)kvh)
                   << logP;
    __syncthreads();
    // A operand of tile t: the query rows 4t .. 4t + 3 (this lane's row is lane & 15), zero
    // elsewhere, so that the four tiles of a group accumulate into one result
    v8i_t qa[4];
    {
        const uint4 *src =
            reinterpret_cast<const uint4 *>(p.qa + (size_t)(bh0 + (lane & 3)) * kD + 32 * (lane >> 4));
        const uint4 a0 = src[0], a1 = src[1];
        const v8i_t q8 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        const int rt = (lane & 15) >> 2;
#pragma unroll
        for (int t = 0; t < 4; ++t) qa[t] = rt == t ? q8 : v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
    float c0[GB], c1[GB];  // wave-uniform
    v4f_t msu;             // -sumu of head h in row h (mod 4): the accumulator input
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        const float4 pq = p.qpar[bh0 + h];
        c0[h] = pq.x;
        c1[h] = pq.y;
        msu[h] = pq.w;
    }
    uint32_t slot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t0 + min(lane + 64 * u, n - 1);
        slot[u] = pbase[(t >> logP) - p0] + (uint32_t)(t & ((1 << logP) - 1));
    }
    uint4 kb[U];
    uint32_t nc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_key_t<KW>(p.c, slot[u], kb[u], nc[u]);
    __builtin_amdgcn_sched_barrier(0);
    int e[U][GB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int pc = __builtin_popcount(kb[u].x) + __builtin_popcount(kb[u].y) + __builtin_popcount(kb[u].z) +
                       __builtin_popcount(kb[u].w);
        const float fP = (float)(2 * pc - 32 * KW);
        const float r = norm_over_corr(nc[u]);
        const v4f_t d = key_products4(kb[u], msu, [&](int t) { return qa[t]; });
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const float a = d[h];
            const float cp = c0[h] * fP;
            const float s = fmaf(c1[h], a, cp) * r;
            e[u][h] = score_bin(s, p.kbin);
        }
    }
    if (n < CH) {  // uniform: the last chunk of a sequence; positions past the end sit below all
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < GB; ++h)
                if (lane + 64 * u >= n) e[u][h] = kNone;
    }
    int lm[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        int m = e[0][h];
#pragma unroll
        for (int u = 1; u < U; ++u) m = max(m, e[u][h]);
        lm[h] = wave_max_iu(m);
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GB; ++h) p.lmax[(size_t)(bh0 + h) * g.NC + chunk] = lm[h];
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        uint16_t *row = p.dl + (size_t)(bh0 + h) * g.Lpad + t0 + lane;
#pragma unroll
        for (int u = 0; u < U; ++u) row[64 * u] = (uint16_t)min(lm[h] - e[u][h], kBins);
    }
}

// Bins of caller-supplied scores (kv_topp_select): one block per (chunk, query head, seq).
__global__ __launch_bounds__(256) void k_bin_scores(BinScoresParams p)
{
    __shared__ int ebuf[8192];
    __shared__ int red[4];
    __shared__ int emax_s[1];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const size_t bh = (size_t)b * g.Hq + h;
    int lm[1] = {-kBinClamp};
    for (int tl = threadIdx.x; tl < n; tl += kBlock) {
        const int e = score_bin(p.scores[bh * g.ld + t0 + tl], p.kbin);
        ebuf[tl] = e;
        lm[0] = max(lm[0], e);
    }
    block_reduce<1>(lm, red, emax_s, MaxI());
    if (threadIdx.x == 0) p.lmax[bh * g.NC + chunk] = emax_s[0];
    for (int tl = threadIdx.x; tl < n; tl += kBlock)
        p.dl[bh * g.Lpad + t0 + tl] = (uint16_t)min(emax_s[0] - ebuf[tl], kBins);
}

// ---------------------------------------------------------------------------------------
// Histogram pass: per (split, query head, sequence) block, counts of tokens per bin
// distance d = (e_max - chunk top) + distance-to-chunk-top, d < 8192, in LDS (atomics), then
// written as 16-bit counts.  1024 threads (16 waves) per block: the pass is latency-bound,
// and more waves per SIMD hide the distance loads.  The threshold pass follows.
// ---------------------------------------------------------------------------------------
constexpr int kHistThreads = 1024;

__global__ __launch_bounds__(kHistThreads) void k_hist(HistParams p)
{
    constexpr int kT = kHistThreads;
    // one 16-byte load per thread and round (8192 tokens), the next round's load in flight
    // while this round is counted (more loads per round, counted after they all arrive,
    // left the atomics and the stream to run one after the other)
    constexpr int U = 1;
    __shared__ uint32_t hist[kBins];
    __shared__ int delta[kT];
    __shared__ int red[kT / 64];
    const DecodeGeom &g = p.g;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t bh = (size_t)b * g.Hq + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (p.order_ctr && (split | h | b | tid) == 0) {
        // the threshold pass, which follows, takes the dispatch-order slots from these
        p.order_ctr[0] = 0;
        p.order_ctr[1] = 0;
    }
    const int L = g.seq_lens[b];
    const int nch = L > 0 ? (L + g.CH - 1) >> g.logCH : 0;
    const int c0 = split * p.cps;
    if (c0 >= nch) return;  // the threshold pass reads only the splits that hold tokens
    const int c1 = min(nch, c0 + p.cps);
    const int tb = c0 << g.logCH;
    const int te = min(L, c1 << g.logCH);
    const uint16_t *row = p.dl + bh * g.Lpad;
    // 8 tokens per 16-byte load (tb is a multiple of CH >= 256).  The first round is issued
    // before the top-bin reduction, whose reads then overlap it.
    constexpr int kStep = 8 * kT * U;
    uint4 raw[U];
    int t = tb + 8 * tid;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (t + 8 * kT * u < te) raw[u] = *reinterpret_cast<const uint4 *>(row + t + 8 * kT * u);
    // the split's chunk top bins, one per thread (the plan keeps cps * CH <= 65535 with
    // CH >= 256, so cps < 256 <= kT), and the chunk top bins of the whole sequence for e_max
    const int lmc = tid < c1 - c0 ? p.lmax[bh * g.NC + c0 + tid] : 0;
    int m = -kBinClamp;
    for (int c = tid; c < nch; c += kT) m = max(m, p.lmax[bh * g.NC + c]);
    for (int i = tid; i < kBins; i += kT) hist[i] = 0u;
    m = wave_max_i(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    int emax = red[0];
#pragma unroll
    for (int w = 1; w < kT / 64; ++w) emax = max(emax, red[w]);
    if (tid < c1 - c0) delta[tid] = emax - lmc;
    __syncthreads();
    for (; t < te; t += kStep) {
        // the next round's loads go out before this round's counting
        uint4 nxt[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (t + kStep + 8 * kT * u < te) nxt[u] = *reinterpret_cast<const uint4 *>(row + t + kStep + 8 * kT * u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tu = t + 8 * kT * u;
            if (tu < te) {
                const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
                const int dc = delta[(tu >> g.logCH) - c0];  // 8 tokens share a chunk
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // tokens past the last bin have no weight and are not counted (sending them
                    // all to one spare counter made it a hot spot when many fall there)
                    const int d = dc + (int)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                    if (tu + e < te && d < kBins) atomicAdd(&hist[d], 1u);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = nxt[u];
    }
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(p.hist + (bh * p.nsplit + split) * kBins);
    for (int i = tid; i < kBins / 8; i += kT) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = hist[8 * i + 2 * q] | (hist[8 * i + 2 * q + 1] << 16);
        dst[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Attention chunks that one wave of a Top-p head covers (log2): 4 or 2 when the head's kept
// count puts at most one batch (64 entries) in such a wave, else 1.  Most heads keep a few
// tokens per chunk; one wave over several chunks then replaces waves whose fixed work (the
// list, the scan, the final sums, the partial) would outweigh their few entries.
__device__ __forceinline__ int attend_span_log2(int kept, int L)
{
    const long e = (long)kept * kTopPAttendChunk, cap = 64L * L;
    return 4 * e <= cap ? 2 : (2 * e <= cap ? 1 : 0);
}

// Dispatch order of the Top-p attention pass: a head whose waves cover one chunk each (the
// dense heads, whose waves work through several dependent batches) takes a slot from the
// front of `order`, any other head one from the back, so that the dense heads' waves start
// first instead of after every head ahead of them in index order.  An entry is the head
// b * Hq + h with log2 of its span in bits 24 and up.  The slots of one class follow the
// order of their atomics; every wave writes the partials of its own (head, chunks), so the
// results do not depend on it.
__device__ __forceinline__ void order_head(const HistParams &p, size_t bh, int kept, int L)
{
    const int BH = p.g.B * p.g.Hq;
    const int ls = attend_span_log2(kept, L);
    const bool dense = ls == 0;
    const int k = atomicAdd(&p.order_ctr[dense ? 0 : 1], 1);
    const int slot = dense ? k : BH - 1 - k;
    if (slot >= 0 && slot < BH) p.order[slot] = (int)bh | (ls << 24);
}

// The threshold of head bh from its bin counts (thread t: bins 8t .. 8t + 7), e_max and the
// sequence length L > 0, in a 1024-thread block: the weighted block scan and the writes
// described at k_thresh.  T holds the 256 weights (published by a barrier before the call);
// wsum, csum and imax are block scratch, imax already holding each wave's top bin.
__device__ __forceinline__ void thresh_finish(const HistParams &p, size_t bh, int L, const uint32_t (&cnt)[8],
                                              const uint64_t *T, uint64_t *wsum, int *csum, const int *imax)
{
    constexpr int kT = 1024;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // d >> 8 is the same for all 8 bins of a thread
    const int shift = tid >> 5;
    uint64_t mine = 0;
    int cmine = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        mine += (uint64_t)cnt[k] * (T[(8 * tid + k) & 255] >> shift);
        cmine += (int)cnt[k];
    }
    uint64_t incl = mine;
    int cincl = cmine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o);
        const int cy = __shfl_up(cincl, o);
        if (lane >= o) {
            incl += y;
            cincl += cy;
        }
    }
    if (lane == 63) {
        wsum[wave] = incl;
        csum[wave] = cincl;
    }
    __syncthreads();
    uint64_t before = incl - mine, Z = 0;
    int cbefore = cincl - cmine, emax = -kBinClamp;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) {
        Z += wsum[w];
        emax = max(emax, imax[w]);
        if (w < wave) {
            before += wsum[w];
            cbefore += csum[w];
        }
    }
    const uint64_t lo = Z * (uint64_t)p.pfx;
    uint64_t hi = __umul64hi(Z, (uint64_t)p.pfx);
    const uint64_t lo2 = lo + ((1ull << 24) - 1);
    hi += (lo2 < lo) ? 1 : 0;
    const uint64_t Tp = (hi << 40) | (lo2 >> 24);
    int bstar = -2, count = 0;  // -2: this thread writes nothing
    if (Tp == 0) {
        if (tid == 0) {
            bstar = 0;
            count = (int)cnt[0];
        }
    } else if (before < Tp && before + mine >= Tp) {
        uint64_t F = before;
        count = cbefore;
        bstar = 8 * tid + 7;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            F += (uint64_t)cnt[k] * (T[(8 * tid + k) & 255] >> shift);
            count += (int)cnt[k];
            if (F >= Tp) {
                bstar = 8 * tid + k;
                break;
            }
        }
    }
    if (emax == -kBinClamp) {
        // every score NaN or at the bottom clamp (for instance records of tokens held in the
        // high-precision tier): no token has weight, the set is empty
        bstar = tid == 0 ? -1 : -2;
        count = 0;
    }
    if (bstar >= -1) {
        if (p.order) order_head(p, bh, count, L);
        p.sel[bh * 4 + 0] = emax;
        p.sel[bh * 4 + 1] = bstar;
        p.sel[bh * 4 + 2] = count;
        if (p.dbg_count) p.dbg_count[bh] = count;
        if (p.dbg_bins) {
            p.dbg_bins[bh * 2] = emax;
            p.dbg_bins[bh * 2 + 1] = bstar;
        }
    }
}

// Top-p threshold of each (b, h) from the split counts: one 1024-thread block per (query
// head, sequence), thread t owns bins 8t .. 8t+7.  A kernel of its own, so that the split
// counts reach it through the kernel boundary rather than through device-scope fences in
// every histogram block.  With W(d) = T[d mod 256] >> (d / 256), T[j] = round(2^(32 - j/256)):
//   Z = sum_d cnt[d] W(d),  T_p = ceil(Z * pfx / 2^24),
//   b* = min { b : sum_{d <= b} cnt[d] W(d) >= T_p },  count = sum_{d <= b*} cnt[d].
// One block scan carries both the weighted sums and the counts, so the thread whose bins
// hold b* writes the result without a further pass.
__global__ __launch_bounds__(1024) void k_thresh(HistParams p)
{
    constexpr int kT = 1024;
    __shared__ uint64_t T[256];
    __shared__ uint64_t wsum[kT / 64];
    __shared__ int csum[kT / 64];
    __shared__ int imax[kT / 64];
    const DecodeGeom &g = p.g;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)b * g.Hq + h;
    // counts of bins 8 tid .. 8 tid + 7 summed over the splits (8 splits' loads in flight).
    // The first 8 splits and the top bins of the first 1024 chunks are read within the
    // planned bounds before the length is known; splits and chunks past it are masked below.
    const uint4 *src = reinterpret_cast<const uint4 *>(p.hist + bh * p.nsplit * kBins) + tid;
    uint4 v0[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v0[k] = k < p.nsplit ? src[(size_t)k * (kBins / 8)] : make_uint4(0u, 0u, 0u, 0u);
    const int mfirst = tid < g.NC ? p.lmax[bh * g.NC + tid] : -kBinClamp;
    // the weight table, while those loads are in flight (published by the barrier below)
    if (tid < 256) T[tid] = (uint64_t)rint(ldexp(exp2(-(double)tid / 256.0), 32));
    const int L = g.seq_lens[b];
    if (L <= 0) {
        if (tid == 0) {
            if (p.order) order_head(p, bh, 0, 0);
            p.sel[bh * 4 + 0] = 0;
            p.sel[bh * 4 + 1] = -1;
            p.sel[bh * 4 + 2] = 0;
            if (p.dbg_count) p.dbg_count[bh] = 0;
            if (p.dbg_bins) {
                p.dbg_bins[bh * 2] = 0;
                p.dbg_bins[bh * 2 + 1] = -1;
            }
        }
        return;
    }
    const int nch = (L + g.CH - 1) >> g.logCH;
    const int nsu = (nch + p.cps - 1) / p.cps;  // splits that hold tokens
    int m = tid < nch ? mfirst : -kBinClamp;
    uint32_t cnt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) cnt[k] = 0u;
    for (int s0 = 0; s0 < nsu; s0 += 8) {
        uint4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (s0 == 0) v[k] = k < nsu ? v0[k] : make_uint4(0u, 0u, 0u, 0u);
            else v[k] = (s0 + k < nsu) ? src[(size_t)(s0 + k) * (kBins / 8)] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cnt[2 * q] += w[q] & 0xFFFFu;
                cnt[2 * q + 1] += w[q] >> 16;
            }
        }
    }
    for (int c = tid + kT; c < nch; c += kT) m = max(m, p.lmax[bh * g.NC + c]);
    m = wave_max_i(m);
    if (lane == 0) imax[wave] = m;
    __syncthreads();
    thresh_finish(p, bh, L, cnt, T, wsum, csum, imax);
}

// ---------------------------------------------------------------------------------------
// Histogram and threshold in one kernel, for heads whose sequence has at most 1024 score
// chunks when there are enough heads to give each a block: the block counts every token of
// its head in LDS (four 16-byte loads per thread and round, the next round's in flight) and
// runs the threshold scan of k_thresh on those counts, so that no split counts go through
// HBM and no second launch is needed.  The dispatch slots were cleared by the query pass.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kHistThreads) void k_hist_thresh(HistParams p)
{
    constexpr int kT = kHistThreads, U = 4;
    constexpr int kStep = 8 * kT * U;  // tokens per round
    __shared__ uint32_t hist[kBins];
    __shared__ int delta[kT];
    __shared__ uint64_t T[256];
    __shared__ uint64_t wsum[kT / 64];
    __shared__ int csum[kT / 64];
    __shared__ int imax[kT / 64];
    const DecodeGeom &g = p.g;
    const int h = blockIdx.x, b = blockIdx.y;
    const size_t bh = (size_t)b * g.Hq + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = g.seq_lens[b];
    const uint16_t *row = p.dl + bh * g.Lpad;
    // the first round's distances (the row holds whole chunks: reads up to Lpad stay in it;
    // tokens past L are not counted) and the chunk top bins, issued together
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = 8 * tid + 8 * kT * u;
        raw[u] = t < g.Lpad ? *reinterpret_cast<const uint4 *>(row + t) : make_uint4(0u, 0u, 0u, 0u);
    }
    const int nch = L > 0 ? (L + g.CH - 1) >> g.logCH : 0;  // <= kT (the plan's condition)
    const int lmc = tid < nch ? p.lmax[bh * g.NC + tid] : -kBinClamp;
    if (tid < 256) T[tid] = (uint64_t)rint(ldexp(exp2(-(double)tid / 256.0), 32));
    for (int i = tid; i < kBins; i += kT) hist[i] = 0u;
    const int m = wave_max_i(lmc);
    if (lane == 0) imax[wave] = m;
    __syncthreads();
    if (L <= 0) {  // uniform
        if (tid == 0) {
            if (p.order) order_head(p, bh, 0, 0);
            p.sel[bh * 4 + 0] = 0;
            p.sel[bh * 4 + 1] = -1;
            p.sel[bh * 4 + 2] = 0;
            if (p.dbg_count) p.dbg_count[bh] = 0;
            if (p.dbg_bins) {
                p.dbg_bins[bh * 2] = 0;
                p.dbg_bins[bh * 2 + 1] = -1;
            }
        }
        return;
    }
    int emax = imax[0];
#pragma unroll
    for (int w = 1; w < kT / 64; ++w) emax = max(emax, imax[w]);
    if (tid < nch) delta[tid] = emax - lmc;
    __syncthreads();
    for (int t = 8 * tid; t < L; t += kStep) {
        uint4 nxt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tn = t + kStep + 8 * kT * u;
            if (tn < L) nxt[u] = *reinterpret_cast<const uint4 *>(row + tn);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tu = t + 8 * kT * u;
            if (tu < L) {
                const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
                const int dc = delta[tu >> g.logCH];  // 8 tokens share a chunk
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = dc + (int)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                    if (tu + e < L && d < kBins) atomicAdd(&hist[d], 1u);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = nxt[u];
    }
    __syncthreads();
    uint32_t cnt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) cnt[k] = hist[8 * tid + k];
    thresh_finish(p, bh, L, cnt, T, wsum, csum, imax);
}

// Bin-distance threshold of a chunk: token kept when its distance to the chunk top bin is
// <= b* - (e_max - chunk top).
__device__ __forceinline__ int chunk_threshold(const int32_t *sel, const int32_t *lmax, size_t bh, int NC,
                                               int chunk)
{
    const int emax = sel[bh * 4 + 0], bstar = sel[bh * 4 + 1];
    const long thr = (long)bstar - ((long)emax - (long)lmax[bh * NC + chunk]);
    return thr < -1 ? -1 : (int)thr;
}

// ---------------------------------------------------------------------------------------
// Ordered selection output: per chunk count, then ascending indices at the chunk's offset.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sel_count(SelectParams p)
{
    __shared__ int red[4];
    __shared__ int tot[1];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t bh = (size_t)b * g.Hq + h;
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int thr = chunk_threshold(p.sel, p.lmax, bh, g.NC, chunk);
    int c[1] = {0};
    for (int tl = threadIdx.x; tl < n; tl += kBlock) c[0] += ((int)p.dl[bh * g.Lpad + t0 + tl] <= thr) ? 1 : 0;
    block_reduce<1>(c, red, tot, SumI());
    if (threadIdx.x == 0) p.cnt[bh * g.NC + chunk] = tot[0];
}

__global__ __launch_bounds__(256) void k_sel_write(SelectParams p)
{
    __shared__ int red[4];
    __shared__ int tot[1];
    __shared__ int wcnt[4];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t bh = (size_t)b * g.Hq + h;
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int o[1] = {0};
    for (int c = threadIdx.x; c < chunk; c += kBlock) o[0] += p.cnt[bh * g.NC + c];
    block_reduce<1>(o, red, tot, SumI());
    int base = tot[0];
    const int thr = chunk_threshold(p.sel, p.lmax, bh, g.NC, chunk);
    for (int tb = 0; tb < n; tb += kBlock) {
        const int tl = tb + threadIdx.x;
        const bool keep = tl < n && (int)p.dl[bh * g.Lpad + t0 + tl] <= thr;
        const uint64_t m = __ballot(keep);
        if (lane == 0) wcnt[wave] = __popcll(m);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wcnt[w];
        if (keep) p.idx[bh * g.ld + off + __popcll(m & lanemask_lt())] = t0 + tl;
        base += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
// Full-softmax attention: one wave per (chunk of CH tokens, KV head, sequence) and GB <= 4
// query heads of that KV head.  The chunk is walked in batches of 64 tokens.  For a batch
// every load is issued up front: one key record per lane (the lane's token) and, per 16-lane
// group, the value words of 16 tokens (4 bytes of codes, i.e. 8 dims, and the group's
// scale/zero word per lane).  The lane scores its token for the GB heads (binary x INT4).
// Each head keeps a reference score m, which moves (a wave max, the earlier batches
// rescaled) only when a score passes it by 8 / (log2e/sqrt(D)); the weights
// exp2((s - m) log2e/sqrt(D)) <= 2^8 go through LDS, and each lane accumulates weight x
// decoded value for its 8 dims (the zero point once per token).  The wave writes (m, sum of
// weights, weighted value sums) per head for the merge.  Used where the matrix-core form
// below would fill fewer than 4 of its 16 rows (one head over 64-dim groups).
// ---------------------------------------------------------------------------------------
template <int GB, int GV, int KW, bool PAGE64>
__global__ __launch_bounds__(64) void k_attend_full(AttendParams p)
{
    static_assert(GB == 1, "the vector-unit pass serves one query head per KV head");
    constexpr int NB = 64;        // tokens per batch
    constexpr int VU = NB / 16;   // value tokens per 4-lane group and batch
    constexpr int VREC = kD / 2 + 4 * (kD / GV);  // bytes of a value record
    __shared__ float wbuf[NB][GB];
    __shared__ uint32_t pbase[kMaxFullChunk / 16 + 1];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int lane = threadIdx.x;
    const int bh0 = b * g.Hq + hq0;
    const int logP = p.c.logP;
    const int p0 = t0 >> logP;
    const int np = ((t0 + n - 1) >> logP) - p0 + 1;
    for (int i = lane; i < np; i += 64)
        pbase[i] = ((uint32_t)g.page_table[(size_t)b * g.max_pages + p0 + i] * (uint32_t)p.c.Hkv + (uint32_t)kvh)
                   << logP;
    QueryState<GB> qs;  // wave-uniform: scalar loads into SGPRs
#pragma unroll
    for (int h = 0; h < GB; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) qs.nib[h][i] = p.qnib[(size_t)(bh0 + h) * 16 + i];
        const float4 pq = p.qpar[bh0 + h];
        qs.c0[h] = pq.x;
        qs.c1[h] = pq.y;
        qs.sumu[h] = __float_as_int(pq.z);
    }
    __syncthreads();

    // values: 4 lanes per token, 32 dims each (one 16-byte load of codes and the group's
    // scale/zero word), so that the per-token scale work is shared by 32 dims and a batch
    // takes 8 value loads per lane
    const int q4 = lane & 3;   // dims 32*q4 .. 32*q4+31
    const int eg = lane >> 2;  // value tokens eg + 16 u of a batch
    const int grp = (32 * q4) / GV;
    const uint32_t tmask = (1u << logP) - 1u;
    const int vw = 16 * q4, vz = kD / 2 + 4 * grp;  // offsets of the lane's codes and scale/zero word
    float acc[GB][32], zacc[GB], lsum[GB], mrun[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        zacc[h] = 0.0f;
        lsum[h] = 0.0f;
        mrun[h] = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[h][j] = 0.0f;
    }

    const float lazy = 8.0f / p.klog;  // score units of a factor 2^8 in weight
    for (int bs = 0; bs < n; bs += NB) {
        const int nb = min(NB, n - bs);
        // ---- the batch's key and value records (the slow path re-reads the last token for
        // those past nb)
        uint4 kb;
        uint32_t nc;
        uint4 cw[VU];
        uint32_t szw[VU];
        if constexpr (PAGE64) {
            // pages of 64 tokens or more hold a whole batch: consecutive slots, one address per
            // lane and fixed offsets; slots past the sequence's end get no weight, and their
            // scale/zero words are cleared so that whatever they hold stays out of the sums
            const uint32_t first = (uint32_t)(t0 + bs);
            const uint32_t s0 = pbase[(first >> logP) - p0] + (first & tmask);
            load_key_t<KW>(p.c, s0 + lane, kb, nc);
            const uint8_t *vr = p.c.vals + (size_t)(s0 + eg) * VREC;
#pragma unroll
            for (int u = 0; u < VU; ++u) {  // 16 tokens further per u
                __builtin_memcpy(&cw[u], vr + (size_t)u * 16 * VREC + vw, 16);  // 8-byte aligned when Gv = 64
                szw[u] = *reinterpret_cast<const uint32_t *>(vr + (size_t)u * 16 * VREC + vz);
            }
            if (nb < NB) {  // uniform: the sequence's last batch
#pragma unroll
                for (int u = 0; u < VU; ++u)
                    if (eg + 16 * u >= nb) szw[u] = 0u;
            }
        } else {
            {
                const uint32_t t = (uint32_t)(t0 + bs + min(lane, nb - 1));
                load_key_t<KW>(p.c, pbase[(t >> logP) - p0] + (t & tmask), kb, nc);
            }
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                const uint32_t t = (uint32_t)(t0 + bs + min(eg + 16 * u, nb - 1));
                const uint8_t *vr = p.c.vals + (size_t)(pbase[(t >> logP) - p0] + (t & tmask)) * VREC;
                __builtin_memcpy(&cw[u], vr + vw, 16);
                szw[u] = *reinterpret_cast<const uint32_t *>(vr + vz);
            }
        }
        float s[GB];
        {
            int A[GB];
            score_key<GB>(kb, nc, qs, s, A, 32 * KW);
        }
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            // past the batch, or a marked record (a token held in the high-precision tier)
            if (lane >= nb || s[h] != s[h]) s[h] = -INFINITY;
            // the reference score moves only when a score passes it by 8 / klog (weights stay
            // <= 2^8), then to the batch max with the partial sums rescaled
            if (__any(s[h] > mrun[h] + lazy)) {
                const float mnew = wave_max_u(s[h]);
                const float scale = (mrun[h] == -INFINITY) ? 0.0f : exp2f((mrun[h] - mnew) * p.klog);
                zacc[h] *= scale;
                lsum[h] *= scale;
#pragma unroll
                for (int j = 0; j < 32; ++j) acc[h][j] *= scale;
                mrun[h] = mnew;
            }
            const float w = (mrun[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((s[h] - mrun[h]) * p.klog);
            lsum[h] += w;
            wbuf[lane][h] = w;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int e = eg + 16 * u;  // weight 0 past nb
            const float sf = half_bits_to_float(szw[u] & 0xFFFFu);
            const float zf = half_bits_to_float(szw[u] >> 16);
            const uint32_t cwk[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll
            for (int h = 0; h < GB; ++h) {
                const float w = wbuf[e][h];
                const float ws = w * sf * kCodeUnscale;  // exact: by 2^9
                zacc[h] = fmaf(w, zf, zacc[h]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {  // word k: dims 32 q4 + 8k .. + 7
                    float c[8];
                    unpack_codes_e4m3(cwk[k], c);  // c * 2^-9
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[h][8 * k + j] = fmaf(ws, c[j], acc[h][8 * k + j]);
                }
            }
        }
        __syncthreads();  // wbuf is rewritten by the next batch
    }

    // ---- weight sums, then the value sums over the 16 token groups (lanes q4, q4 + 4, ...)
    const size_t pidx = (size_t)bh0 * g.NCA + chunk;  // partial of head bh0 (+ h * NCA)
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        const float l = wave_sum(lsum[h]);
#pragma unroll
        for (int o = 4; o < 64; o <<= 1) {
            zacc[h] += xor_lane(zacc[h], o);
#pragma unroll
            for (int j = 0; j < 32; ++j) acc[h][j] += xor_lane(acc[h][j], o);
        }
        if (lane < 4) {
            float4 *dst = reinterpret_cast<float4 *>(p.po + (pidx + (size_t)h * g.NCA) * kD + 32 * lane);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                dst[k] = make_float4(acc[h][4 * k] + zacc[h], acc[h][4 * k + 1] + zacc[h], acc[h][4 * k + 2] + zacc[h],
                                     acc[h][4 * k + 3] + zacc[h]);
        }
        if (lane == 0) {
            p.pm[pidx + (size_t)h * g.NCA] = mrun[h];
            p.pl[pidx + (size_t)h * g.NCA] = l;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Full-softmax attention with the weighted value sums on the matrix cores.  One wave per
// (chunk of CH tokens, KV head, sequence) and GB <= 4 query heads of that KV head, batches of
// 64 tokens as two steps of 32 through v_mfma_f32_16x16x32_bf16:
//   O[(h, g)][d] = sum_t A[(h, g)][t] B[t][d],  A = w_h(t) * scale_g(t),  B = code_d(t),
// with the A rows (h, g) = NG h + g (NG = 128 / GV groups; rows past GB heads are zero) and
// the dims in 8 tiles of 16 columns (tile j, column n: dim 8n + j); a row keeps the dims of
// its own group.
//  - A goes in as a bfloat16 pair hi + lo (A - hi - lo within 2^-18 A), both through the
//    MFMA against the same B.
//  - B holds the 4-bit code c as the bfloat16 128 + c (bits 0x4300 | c, exact): one byte
//    permute and one and-or per two codes.  A ninth tile with B = 128 gives 128 * sum_t A per
//    row, subtracted at the end; fp32 accumulation keeps the sum to about 2^-19 relative.
//  - the zero points add sum_t w_h(t) zero_g(t) per row, in fp32 on the vector unit.
// Lane l scores token l of the batch (binary x INT4; for four heads on the matrix cores as in
// k_score_topp_mf, with the query operand read from LDS per tile).  As an A row it is
// (h, g) = l mod 16, as a B column the dims 8 (l mod 16) .. + 7, and in both roles it covers
// tokens 8 (l / 16) .. + 7 of each 32-token step; so per token of that K block it loads the
// 4 code bytes of its dims and the scale/zero word of its row's group, and reads the weights
// of its row's head from LDS.  Output rows 4 (l / 16) + i, columns l mod 16 (the MFMA's
// accumulator layout): lane l ends with 8 dims of the heads whose group matches its dims.
// The softmax keeps a reference score per head as k_attend_full does.
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// x0, x1 rounded to bfloat16 (hi) and the rounded remainders (lo), two per word, x0 low
__device__ __forceinline__ void bf16_split2(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    const bf16x2_t h = __builtin_convertvector((f2_t){x0, x1}, bf16x2_t);
    __builtin_memcpy(&hi, &h, 4);
    const f2_t r = {x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u)};
    const bf16x2_t l = __builtin_convertvector(r, bf16x2_t);
    __builtin_memcpy(&lo, &l, 4);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const uint4 v = make_uint4(a, b, c, d);
    bf16x8_t r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ float pick4(const v4f_t &v, int i)
{
    return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// A wave-uniform value (loaded by every lane from one address) moved to a scalar register.
__device__ __forceinline__ float uniform_f(float v)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// LDS ordering among the lanes of one wave (for data no other wave touches): a wave's LDS
// operations complete in order, so fences at wavefront scope, which keep the compiler from
// moving LDS accesses across this point, are all that is needed.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave's state of the matrix-core pass: the 9 accumulator tiles, the zero-point sum of the
// lane's A row, and per head the lane's weight sum and the (wave-uniform) reference score.
template <int GB>
struct MfState {
    v4f_t acc[9];
    float zacc, lsum[GB], mrun[GB];
};

// LDS of one wave of the pass: the batch's weights by head (row GB stays zero: the A rows of
// heads past GB read it), the 4 heads' fp8 query codes and 32 zero bytes, the page ids of the
// pass's tokens (NPB entries: tokens / 16 + 1 for pages of >= 16 tokens).
template <int GB, int NPB>
struct MfShared {
    float wbuf[GB + 1][64];
    uint4 qa[34];
    uint32_t pbase[NPB];
};

// The matrix-core pass of one wave over tokens tb .. tb + n - 1 of sequence b for the GB query
// heads bh0 .. of KV head kvh (the scheme above).  MASKED (Top-p): a token counts for head h
// only if the Top-p bin of its score is at least ebin[h] = e_max - b* of the head (the score
// is the score pass's, bit for bit, so this is the set the threshold pass counted).  Leaves
// the sums in st; mf_outputs gives the value sums.
template <int GB, int GV, int KW, bool PAGE64, bool MASKED, int NPB>
__device__ __forceinline__ void mf_pass(const AttendParams &p, int b, int kvh, int bh0, int tb, int n,
                                        MfShared<GB, NPB> &sh, MfState<GB> &st, const int *ebin = nullptr)
{
    constexpr int NB = 64;                // tokens per batch
    constexpr int NG = kD / GV;           // value groups per token
    constexpr int VREC = kD / 2 + 4 * NG;  // bytes of a value record
    static_assert(GB * NG <= 16, "A rows");
    constexpr bool MF4 = GB == 4;  // four heads: the key products on the matrix cores as well
    const DecodeGeom &g = p.g;
    const int lane = threadIdx.x & 63;
    const int logP = p.c.logP;
    const int p0 = tb >> logP;
    const int np = ((tb + n - 1) >> logP) - p0 + 1;
    for (int i = lane; i < np; i += 64)
        sh.pbase[i] = ((uint32_t)g.page_table[(size_t)b * g.max_pages + p0 + i] * (uint32_t)p.c.Hkv + (uint32_t)kvh)
                      << logP;
    sh.wbuf[GB][lane] = 0.0f;
    QueryState<MF4 ? 1 : GB> qs;  // wave-uniform: scalar loads into SGPRs (dot8 products)
    // per head (wave-uniform, held in scalar registers): the score coefficients and -sumu,
    // which is added to the matrix-core products (integers below 2^24: exact either way)
    float c0[GB], c1[GB], msu[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        const float4 pq = p.qpar[bh0 + h];
        c0[h] = uniform_f(pq.x);
        c1[h] = uniform_f(pq.y);
        msu[h] = 0.0f;
        if constexpr (MF4) {
            msu[h] = uniform_f(pq.w);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) qs.nib[h][i] = p.qnib[(size_t)(bh0 + h) * 16 + i];
            qs.c0[h] = pq.x;
            qs.c1[h] = pq.y;
            qs.sumu[h] = __float_as_int(pq.z);
        }
    }
    if constexpr (MF4) {
        if (lane < 32) sh.qa[lane] = reinterpret_cast<const uint4 *>(p.qa + (size_t)bh0 * kD)[lane];
        else if (lane < 34) sh.qa[lane] = make_uint4(0u, 0u, 0u, 0u);
    }
    wave_lds_sync();
    // A operand of key-product tile t: query head lane & 3 in row lane & 15 of tile
    // (lane & 15) >> 2, its 32 codes of K block lane >> 4; zeros in the other tiles
    const int qrow = 8 * (lane & 3) + 2 * (lane >> 4), qtile = (lane & 15) >> 2;

    const int r16 = lane & 15, kb = lane >> 4;
    const int ha = r16 / NG, ga = r16 % NG;  // the lane's A row
    const int hw = ha < GB ? ha : GB;        // its weight row (the zero row past GB)
    const int vw = 4 * r16;                  // its code word: dims 8 r16 .. 8 r16 + 7
    const int vz = kD / 2 + 4 * ga;          // the scale/zero word of its A row's group
    const uint32_t tmask = (1u << logP) - 1u;
    const uint32_t c128 = 0x43004300u;       // two bfloat16 128s
    const bf16x8_t b128 = as_bf16x8(c128, c128, c128, c128);
#pragma unroll
    for (int j = 0; j < 9; ++j) st.acc[j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    st.zacc = 0.0f;
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        st.lsum[h] = 0.0f;
        st.mrun[h] = -INFINITY;
    }
    const float lazy = 8.0f / p.klog;  // score units of a factor 2^8 in weight

    for (int bs = 0; bs < n; bs += NB) {
        const int nb = min(NB, n - bs);
        // ---- the batch's key and value records
        uint4 kbw;
        uint32_t nc;
        uint32_t cw[16], szw[16];  // entry 8 kt + i: token 32 kt + 8 kb + i of the batch
        if constexpr (PAGE64) {
            // pages of 64 tokens or more hold a whole batch (it starts at a multiple of 64):
            // consecutive slots, one address per lane and fixed offsets.  Slots past the
            // sequence's end are read but get no weight, and their scale/zero words are
            // cleared below, so that whatever they hold stays out of the sums.
            const uint32_t first = (uint32_t)(tb + bs);
            const uint32_t s0 = sh.pbase[(first >> logP) - p0] + (first & tmask);
            load_key_t<KW>(p.c, s0 + lane, kbw, nc);
            const uint8_t *vr = p.c.vals + (size_t)(s0 + 8 * kb) * VREC;
            const uint32_t *cwp = reinterpret_cast<const uint32_t *>(vr + vw);
            const uint32_t *szp = reinterpret_cast<const uint32_t *>(vr + vz);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    cw[8 * kt + i] = cwp[(32 * kt + i) * (VREC / 4)];
                    szw[8 * kt + i] = szp[(32 * kt + i) * (VREC / 4)];
                }
            if (nb < NB) {  // uniform: the sequence's last batch
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (32 * kt + 8 * kb + i >= nb) szw[8 * kt + i] = 0u;
            }
        } else {
            // tokens past nb re-read the last one
            {
                const uint32_t t = (uint32_t)(tb + bs + min(lane, nb - 1));
                load_key_t<KW>(p.c, sh.pbase[(t >> logP) - p0] + (t & tmask), kbw, nc);
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t t = (uint32_t)(tb + bs + min(32 * kt + 8 * kb + i, nb - 1));
                    const uint8_t *vr = p.c.vals + (size_t)(sh.pbase[(t >> logP) - p0] + (t & tmask)) * VREC;
                    cw[8 * kt + i] = *reinterpret_cast<const uint32_t *>(vr + vw);
                    szw[8 * kt + i] = *reinterpret_cast<const uint32_t *>(vr + vz);
                }
        }
        float s[GB];
        if constexpr (MF4) {
            const int pc = __builtin_popcount(kbw.x) + __builtin_popcount(kbw.y) + __builtin_popcount(kbw.z) +
                           __builtin_popcount(kbw.w);
            const float fP = (float)(2 * pc - 32 * KW);
            const float r = norm_over_corr(nc);
            const v4f_t d = key_products4(kbw, v4f_t{0.0f, 0.0f, 0.0f, 0.0f}, [&](int t) {
                const uint4 *q = &sh.qa[qtile == t ? qrow : 32];
                const uint4 a0 = q[0], a1 = q[1];
                return v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            });
#pragma unroll
            for (int h = 0; h < GB; ++h) s[h] = fmaf(c1[h], d[h] + msu[h], c0[h] * fP) * r;
        } else {
            int A[GB];
            score_key<GB>(kbw, nc, qs, s, A, 32 * KW);
        }
        // ---- reference score per head (wave-uniform): the weights are exp2((s - m) klog) <= 2^8.
        // m moves only when a score passes m + 8 / klog, then to the batch max, and the partial
        // sums are rescaled; most batches cost one compare per head instead of a wave max.
        float scl[GB];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            // past the batch, a marked record (a token held in the high-precision tier), or
            // (masked) a token outside the head's Top-p set
            if constexpr (MASKED) {
                if (score_bin(s[h], p.kbin) < ebin[h]) s[h] = -INFINITY;  // NaN: the bottom bin
            }
            if (lane >= nb || s[h] != s[h]) s[h] = -INFINITY;
            scl[h] = 1.0f;
            if (__any(s[h] > st.mrun[h] + lazy)) {  // the first finite score always moves it
                const float mnew = wave_max_u(s[h]);
                scl[h] = (st.mrun[h] == -INFINITY) ? 0.0f : exp2f((st.mrun[h] - mnew) * p.klog);
                st.mrun[h] = mnew;
                grow = true;
            }
        }
        if (grow) {  // wave-uniform
            float f[4];  // accumulator register i holds row 4 kb + i, of head (4 kb + i) / NG
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hr = (4 * kb + i) / NG;
                float v = 1.0f;
#pragma unroll
                for (int h = 0; h < GB; ++h) v = hr == h ? scl[h] : v;
                f[i] = v;
            }
#pragma unroll
            for (int j = 0; j < 9; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) st.acc[j][i] *= f[i];
            float fz = 1.0f;
#pragma unroll
            for (int h = 0; h < GB; ++h) fz = ha == h ? scl[h] : fz;
            st.zacc *= fz;
#pragma unroll
            for (int h = 0; h < GB; ++h) st.lsum[h] *= scl[h];
        }
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            // v_exp_f32 (exp2(-inf) = 0); no weight while the head has no finite score
            const float w = (st.mrun[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((s[h] - st.mrun[h]) * p.klog);
            st.lsum[h] += w;
            sh.wbuf[h][lane] = w;
        }
        wave_lds_sync();
        // ---- two 32-token steps on the matrix cores
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const float4 wa = *reinterpret_cast<const float4 *>(&sh.wbuf[hw][32 * kt + 8 * kb]);
            const float4 wb = *reinterpret_cast<const float4 *>(&sh.wbuf[hw][32 * kt + 8 * kb + 4]);
            const float w8[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sz = szw[8 * kt + i];
                x[i] = w8[i] * half_bits_to_float(sz & 0xFFFFu);
                st.zacc = fmaf(w8[i], half_bits_to_float(sz >> 16), st.zacc);
            }
            uint32_t ah[4], al[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) bf16_split2(x[2 * m], x[2 * m + 1], ah[m], al[m]);
            const bf16x8_t Ahi = as_bf16x8(ah[0], ah[1], ah[2], ah[3]);
            const bf16x8_t Alo = as_bf16x8(al[0], al[1], al[2], al[3]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // byte k of the code words: dims 8 r16 + 2k (low nibble) and + 2k + 1 (high)
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    // byte k of tokens 2m and 2m + 1 into bytes 0 and 2, zeros between
                    const uint32_t q = __builtin_amdgcn_perm(cw[8 * kt + 2 * m + 1], cw[8 * kt + 2 * m],
                                                             0x0C000C00u | ((4u + k) << 16) | (uint32_t)k);
                    lo[m] = and_or(q, 0x000F000Fu, c128);
                    hi[m] = and_or(q >> 4, 0x000F000Fu, c128);
                }
                const bf16x8_t Blo = as_bf16x8(lo[0], lo[1], lo[2], lo[3]);
                const bf16x8_t Bhi = as_bf16x8(hi[0], hi[1], hi[2], hi[3]);
                st.acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, Blo, st.acc[2 * k], 0, 0, 0);
                st.acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, Bhi, st.acc[2 * k + 1], 0, 0, 0);
                st.acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, Blo, st.acc[2 * k], 0, 0, 0);
                st.acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, Bhi, st.acc[2 * k + 1], 0, 0, 0);
            }
            st.acc[8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ahi, b128, st.acc[8], 0, 0, 0);
            st.acc[8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Alo, b128, st.acc[8], 0, 0, 0);
        }
        wave_lds_sync();  // wbuf is rewritten by the next batch
    }
}

// The value sums of a finished pass: out(h, d0, o) receives o[j] = sum_t w_h(t) v_t[d0 + j],
// j < 8, for every head and 8-dim block the lane holds (each (head, block) once in the wave).
// Lane l holds columns l mod 16 (dims 8 (l mod 16) + j of tile j) of rows 4 (l / 16) + i; the
// rows of the dims' own group are i = gd (NG = 4) or i = gd, gd + 2 (NG = 2).
template <int GB, int GV, typename Out>
__device__ __forceinline__ void mf_outputs(MfState<GB> &st, Out out)
{
    constexpr int NG = kD / GV;
    const int lane = threadIdx.x & 63, r16 = lane & 15, kb = lane >> 4;
    // zero-point sums of each A row over its 4 token blocks (lanes r16 + 16 k)
    float z = st.zacc;
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    const int gd = (8 * r16) / GV;
#pragma unroll
    for (int q = 0; q < 4 / NG; ++q) {
        const int i = gd + NG * q;
        const int row = 4 * kb + i, h = row / NG;
        const float zr = __shfl(z, row);  // lanes row, row + 16, ... hold the row's sum
        if (h < GB) {
            const float c = pick4(st.acc[8], i);
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = (pick4(st.acc[j], i) - c) + zr;
            out(h, 8 * r16, o);
        }
    }
}

template <int GB, int GV, int KW, bool PAGE64>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void k_attend_full_mf(AttendParams p)
{
    __shared__ MfShared<GB, kMaxFullChunk / 16 + 1> sh;
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int bh0 = b * g.Hq + hq0;
    MfState<GB> st;
    mf_pass<GB, GV, KW, PAGE64, false>(p, b, kvh, bh0, t0, n, sh, st);
    const size_t pidx = (size_t)bh0 * g.NCA + chunk;  // partial of head bh0 (+ h * NCA)
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        const float l = wave_sum(st.lsum[h]);
        if (threadIdx.x == 0) {
            p.pm[pidx + (size_t)h * g.NCA] = st.mrun[h];
            p.pl[pidx + (size_t)h * g.NCA] = l;
        }
    }
    mf_outputs<GB, GV>(st, [&](int h, int d0, const float (&o)[8]) {
        float4 *dst = reinterpret_cast<float4 *>(p.po + (pidx + (size_t)h * g.NCA) * kD + d0);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    });
}

// ---------------------------------------------------------------------------------------
// Top-p attention: blocks of 4 waves over 4 attention chunks of 1024 tokens of one query
// head, the heads taken in the dispatch order of the threshold pass (dense heads first, each
// with its span).  A dense head's wave covers one chunk; a head that keeps few tokens has one
// wave over 2 or 4 chunks, and the block's other waves end at once.  The waves of a block
// share no data (each has its own LDS slices), so a block holds no barrier.
// Top-p keeps a small, head-specific set of tokens, so the wave first lists the kept tokens
// of its span in ascending order (one pass over the 16-bit bin distances, 8 tokens per
// 16-byte load, one wave scan of packed 16-bit counts), then works through the list in
// batches of 64 entries.  For a batch every load is issued up front: one key record per lane
// and, per 4-lane group, the value records of up to 4 entries (16 bytes of codes, i.e. 32
// dims, and the group's scale/zero word per lane).  Scores, the running max and the weights
// follow, then the weighted value sums from registers.  A chunk that keeps at most 64 tokens
// costs two dependent rounds of HBM reads: the distances (with the query, thresholds and
// page ids), then the kept records.
// Distances past a sequence's end (within its last 512-token score chunk) are 8192, above
// every threshold, so only whole 16-byte groups need a bound check; a group whose smallest
// distance is above the threshold (most of them) costs a few packed 16-bit ops.
// ---------------------------------------------------------------------------------------
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dpp_ror(float v, int k)
{
    // row_ror:k within each 16-lane row (DPP control 0x120 + k); every lane has a source
    const int r = k == 4 ? __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true)
                         : __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true);
    return __int_as_float(r);
}

constexpr int kAttendWaves = 4;  // waves per Top-p attention block: 4 chunks of one head

// ---------------------------------------------------------------------------------------
// Top-p attention of 4 attention chunks (one per wave) for a KV head's 4 query heads that
// each keep more than 1 / kMaskedDense of their sequence.  Gathering the kept records per
// head then reads most records several times over (through the caches) and lists every kept
// token; instead each wave runs the full-softmax matrix-core pass over its chunk with a mask
// (a token counts for a head when the Top-p bin of its score, which the pass recomputes bit
// for bit, is at least the head's e_max - b*), reading every key and value record of the
// chunk once for the 4 heads and none of the bin distances.  The waves' (reference score, weight sum, value sums) per head are combined through
// LDS into one partial per head, written to slot `slot`: the quantities the gather pass
// writes for its chunks, up to rounding.  Chunks past the sequence's end contribute nothing.
// smem: kMaskedSmem bytes, 16-byte aligned; every thread of the block calls it (it holds
// block barriers).
// ---------------------------------------------------------------------------------------
constexpr int kMaskedDense = 4;
constexpr int kMaskedPages = kTopPAttendChunk / 64 + 1;  // page ids of a chunk (pages >= 64)
constexpr int kMaskedSlice = (int)sizeof(MfShared<4, kMaskedPages>);
constexpr int kMaskedCombine = (4 * 4 * kD + 2 * 4 * 4) * 4;  // [wave][head][128] sums, then m and l
constexpr int kMaskedSmem = 4 * kMaskedSlice > kMaskedCombine ? 4 * kMaskedSlice : kMaskedCombine;
static_assert(sizeof(MfShared<4, kMaskedPages>) % 16 == 0, "slices stay 16-byte aligned");

template <int GV, int KW>
__device__ __forceinline__ void topp_masked_chunks(const AttendParams &p, int b, int kvh, int hq0, int c, int slot,
                                                   int L, uint8_t *smem)
{
    constexpr int GB = 4, NW = 4, CHA = kTopPAttendChunk;
    using Sh = MfShared<GB, kMaskedPages>;
    const DecodeGeom &g = p.g;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bh0 = b * g.Hq + hq0;
    const int tb = c * CHA;
    MfState<GB> st;
    if (tb < L) {  // wave-uniform
        uint8_t *slice = smem + kMaskedSlice * wave;
        // the heads' lowest kept bin, e_max - b* (wave-uniform)
        int ebin[GB];
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const int *sl = p.sel + (size_t)(bh0 + h) * 4;
            ebin[h] = __builtin_amdgcn_readfirstlane(sl[0] - sl[1]);
        }
        mf_pass<GB, GV, KW, true, true>(p, b, kvh, bh0, tb, min(CHA, L - tb), *reinterpret_cast<Sh *>(slice), st,
                                        ebin);
    } else {  // past the sequence's end: nothing
#pragma unroll
        for (int j = 0; j < 9; ++j) st.acc[j] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
        st.zacc = 0.0f;
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            st.lsum[h] = 0.0f;
            st.mrun[h] = -INFINITY;
        }
    }
    float l[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) l[h] = wave_sum(st.lsum[h]);
    __syncthreads();  // every wave is done with its LDS slice
    float *cmb = reinterpret_cast<float *>(smem);  // [NW][GB][128] value sums, then [NW][GB] m and l
    float *cm = cmb + NW * GB * kD, *cl = cm + NW * GB;
    mf_outputs<GB, GV>(st, [&](int h, int d0, const float (&o)[8]) {
        float4 *dst = reinterpret_cast<float4 *>(cmb + (wave * GB + h) * kD + d0);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    });
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            cm[wave * GB + h] = st.mrun[h];
            cl[wave * GB + h] = l[h];
        }
    }
    __syncthreads();
    // wave h: head h, lane l: dims 2 l and 2 l + 1
    const int h = wave, d = 2 * lane;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, cm[w * GB + h]);
    float o0 = 0.0f, o1 = 0.0f, lt = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float mw = cm[w * GB + h];
        const float a = (mw == -INFINITY) ? 0.0f : exp2f((mw - M) * p.klog);
        o0 = fmaf(a, cmb[(w * GB + h) * kD + d], o0);
        o1 = fmaf(a, cmb[(w * GB + h) * kD + d + 1], o1);
        lt = fmaf(a, cl[w * GB + h], lt);
    }
    const size_t pidx = (size_t)(bh0 + h) * g.NCA + slot;
    reinterpret_cast<float2 *>(p.po + pidx * kD)[lane] = make_float2(o0, o1);
    if (lane == 0) {
        p.pm[pidx] = M;
        p.pl[pidx] = lt;
    }
}

// Whether the query heads hq0 .. hq0 + 3 of sequence b (a KV head's group) each keep more
// than 1 / kMaskedDense of the sequence's L tokens (the threshold pass's counts).
__device__ __forceinline__ bool masked_group(const AttendParams &p, int b, int hq0, int L)
{
    bool many = true;
#pragma unroll
    for (int h = 0; h < 4; ++h) many &= (long)kMaskedDense * p.sel[(size_t)(b * p.g.Hq + hq0 + h) * 4 + 2] > L;
    return many;
}

// MG: 0, or the value group size (32 or 64) when the masked chunk pass is compiled in (groups
// of 4 query heads, pages of 64 tokens or more, compressed keys).
template <bool EXACT, int KW, int MG>
__global__ __launch_bounds__(64 * kAttendWaves, EXACT ? 1 : 4) void k_attend_topp(AttendParams p)
{
    constexpr int CHA = kTopPAttendChunk;  // tokens of an attention chunk
    constexpr int NW = kAttendWaves;
    constexpr int NJ = CHA * NW / 512;     // 16-byte distance loads per lane, widest span
    constexpr int NB = EXACT ? 32 : 64;    // entries per batch
    constexpr int VU = NB / 16;            // value entries per 4-lane group and batch
    // per-wave slices; a wave over s chunks uses the s slices of its group, contiguous.  A
    // list slice is 2304 bytes so that the final sums (2304 bytes) fit in one.
    constexpr int SL = 1152;               // list entries per slice
    constexpr int PS = CHA / 16 + 1;       // page ids per slice (pages of >= 16 tokens)
    // the list slices; with the masked chunk pass, also the waves' slices of that pass
    constexpr int LST = MG != 0 && kMaskedSmem > NW * SL * 2 ? kMaskedSmem / 2 : NW * SL;
    __shared__ __align__(16) uint16_t lst[LST];
    __shared__ float wbs[NW][64];
    __shared__ uint32_t pbs[NW * PS];
    const DecodeGeom &g = p.g;
    if constexpr (MG != 0) {
        // every head dense, and the block's group of 4 heads each keeping a large share: one
        // read of every record of a chunk for the 4 heads, one chunk per wave.  The block
        // numbering is the dense case's below (block xf of the group's NCA).  Blocks
        // xf < nq = NCA / 4 take chunks xf + nq w (wave w) and write their combined partial to
        // slot xf; the others mark slot xf empty and end, so that the working blocks are
        // consecutive (spread over the XCDs as blocks are dealt out) and the merge finds the
        // partials in the first nq slots.
        static_assert(NW == 4, "masked chunk pass: 4 waves per block");
        if (p.order_ctr[0] == g.B * g.Hq && g.GB == 4) {
            const int L0 = (int)blockIdx.x + (int)gridDim.x * ((int)blockIdx.y + (int)gridDim.y * (int)blockIdx.z);
            const int grp = L0 / g.NCA, xf = L0 - grp * g.NCA;
            if (grp < g.B * g.Hkv * g.nsub) {
                const int bq = grp / (g.Hkv * g.nsub);
                int kvg, hq0;
                block_heads(g, grp - bq * g.Hkv * g.nsub, kvg, hq0);
                const int Lq = g.seq_lens[bq];
                if (masked_group(p, bq, hq0, Lq)) {  // block-uniform
                    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
                    const int nq = (g.NCA + 3) >> 2;
                    if (xf < nq) {
                        topp_masked_chunks<MG, KW>(p, bq, kvg, hq0, xf + nq * w, xf, Lq,
                                                   reinterpret_cast<uint8_t *>(lst));
                    } else if (threadIdx.x < 4) {
                        const size_t pidx = (size_t)(bq * g.Hq + hq0 + threadIdx.x) * g.NCA + xf;
                        p.pm[pidx] = -INFINITY;
                        p.pl[pidx] = 0.0f;
                    }
                    return;
                }
            }
        }
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar
    int bhr, ls, c0, first;
    if (p.order_ctr[0] == g.B * g.Hq) {
        // every head covers its chunks one by one (each keeps many tokens): the blocks are
        // renumbered so that a block holds the GB query heads of one KV head for NW / GB
        // consecutive chunks (wave w: head w mod GB, chunk w / GB).  Those waves run on one
        // compute unit at the same time, so a record that several of the heads keep crosses
        // HBM once and reaches the others from the caches.
        const int GB = g.GB, cpb = NW / GB;
        const int nxf = (g.NCA + cpb - 1) / cpb;
        const int L0 = (int)blockIdx.x + (int)gridDim.x * ((int)blockIdx.y + (int)gridDim.y * (int)blockIdx.z);
        const int grp = L0 / nxf, xf = L0 - grp * nxf;
        const int ngrp = g.B * g.Hkv * g.nsub;
        if (grp >= ngrp) return;
        const int bq = grp / (g.Hkv * g.nsub);
        int kvg, hq0;
        block_heads(g, grp - bq * g.Hkv * g.nsub, kvg, hq0);
        bhr = bq * g.Hq + hq0 + (wave & (GB - 1));
        ls = 0;
        first = wave;
        c0 = xf * cpb + wave / GB;
    } else {
        // the head of this dispatch rank and its span (dense heads first; the threshold pass
        // wrote the order)
        const int code = p.order[blockIdx.z * g.Hq + blockIdx.y];
        bhr = code & 0xFFFFFF;
        ls = (code >> 24) & 3;
        if (bhr >= g.B * g.Hq) bhr = blockIdx.z * g.Hq + blockIdx.y;
        // the block's waves cover chunks NW bx .. + NW - 1, in groups of span = 2^ls; one
        // wave per group works, the one whose index within the group rotates with the block,
        // so that the working waves spread over the SIMDs; the others have nothing to do
        const int sp = 1 << ls;
        first = wave & ~(sp - 1);  // first wave (and slice) of this wave's group
        if (wave - first != ((int)blockIdx.x & (sp - 1))) return;
        c0 = (int)blockIdx.x * NW + first;  // first chunk of the span
    }
    const int b = bhr / g.Hq, h = bhr - b * g.Hq;
    const int kvh = h / g.G;
    const size_t bh = (size_t)bhr;
    const int span = 1 << ls;
    if (c0 >= g.NCA) return;
    const int t0 = c0 * CHA;
    uint16_t *list = lst + first * SL;
    float4(*red)[4][9] = reinterpret_cast<float4(*)[4][9]>(list);  // after the last batch
    float *wbuf = wbs[wave];
    uint32_t *pbase = pbs + first * PS;

    // ---- round 1: the span's distances (tokens 8 lane + 512 j .. + 7), thresholds and page
    // ids, and the sequence length, all issued together: the distance rows hold whole
    // attention chunks and the page ids are read within the table, so none of these loads
    // waits for the length (values past it are masked below)
    // Every load is issued without a branch (a load under a branch made the wave wait for it
    // where the paths join): groups past the span or the padded row re-read the first group,
    // and thresholds past the last score chunk read the last one; both are masked below.
    uint4 raw[NJ];
    int thr[NJ];  // wave-uniform
    const uint16_t *row = p.dl + bh * g.Lpad + t0;
    const int nj = min(span * (CHA / 512), (g.NCA - c0) * (CHA / 512));  // groups in the row
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        raw[j] = *reinterpret_cast<const uint4 *>(row + 8 * lane + 512 * (j < nj ? j : 0));
        const int chunk = c0 * (CHA / 512) + j;
        thr[j] = chunk_threshold(p.sel, p.lmax, bh, g.NC, min(chunk, g.NC - 1));
        if (j >= nj || chunk >= g.NC) thr[j] = -1;
    }
    const int logP = p.c.logP;
    const int p0 = t0 >> logP;
    const int npmax = min(((t0 + CHA * span - 1) >> logP) - p0 + 1, g.max_pages - p0);
    for (int i = lane; i < npmax; i += 64)
        pbase[i] = ((uint32_t)g.page_table[(size_t)b * g.max_pages + p0 + i] * (uint32_t)p.c.Hkv + (uint32_t)kvh)
                   << logP;
    const int L = g.seq_lens[b];
    if (t0 >= L) return;
    const int n = min(CHA * span, L - t0);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        if (j * kTopPChunk >= n) thr[j] = -1;  // a 512-token chunk past the end keeps nothing
    QueryState<1> qs;  // wave-uniform: scalar loads into SGPRs
#pragma unroll
    for (int i = 0; i < 16; ++i) qs.nib[0][i] = p.qnib[bh * 16 + i];
    {
        const float4 qp = p.qpar[bh];
        qs.c0[0] = qp.x;
        qs.c1[0] = qp.y;
        qs.sumu[0] = __float_as_int(qp.z);
    }

    // ---- kept tokens, listed in ascending order
    uint32_t keep[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int tl = 8 * lane + 512 * j;
        uint32_t m = 0u;
        if (tl < n) {
            u16x2 w2[4];
            __builtin_memcpy(w2, &raw[j], 16);
            const u16x2 mn = __builtin_elementwise_min(__builtin_elementwise_min(w2[0], w2[1]),
                                                       __builtin_elementwise_min(w2[2], w2[3]));
            if ((int)min(mn.x, mn.y) <= thr[j]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) m |= ((int)w2[e >> 1][e & 1] <= thr[j]) ? (1u << e) : 0u;
            }
        }
        keep[j] = m;
    }
    // wave-wide inclusive scans of the packed 16-bit counts, four 512-token groups per word
    // (a field never exceeds 512); the second word only for a span of more than two chunks
    uint64_t cnt4[2] = {0, 0}, before[2] = {0, 0}, total[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < NJ; ++j) cnt4[j >> 2] |= (uint64_t)__builtin_popcount(keep[j]) << (16 * (j & 3));
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        if (w == 0 || span > 2) {
            uint64_t incl = cnt4[w];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint64_t y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            total[w] = __shfl(incl, 63);
            before[w] = incl - cnt4[w];
        }
    }
    int nlist = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        int off = nlist + (int)((before[j >> 2] >> (16 * (j & 3))) & 0xFFFFu);
        uint32_t m = keep[j];
        while (m) {
            const int e = __builtin_ctz(m);
            m &= m - 1u;
            list[off++] = (uint16_t)(8 * lane + 512 * j + e);
        }
        nlist += (int)((total[j >> 2] >> (16 * (j & 3))) & 0xFFFFu);
    }
    nlist = __builtin_amdgcn_readfirstlane(nlist);  // wave-uniform: scalar loop control
    wave_lds_sync();

    const int q4 = lane & 3;   // dims 32*q4 .. 32*q4+31
    const int eg = lane >> 2;  // entries eg + 16 u of a batch
    const int grp = (32 * q4) / p.c.Gv;
    const uint32_t tmask = (1u << logP) - 1u;
    // exact scores: this lane's 32 query dims (binary32)
    float qx[EXACT ? 32 : 1];
    if constexpr (EXACT) {
        const float4 *qs4 = reinterpret_cast<const float4 *>(p.q + bh * kD + 32 * q4);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float4 v = qs4[k];
            qx[4 * k] = v.x;
            qx[4 * k + 1] = v.y;
            qx[4 * k + 2] = v.z;
            qx[4 * k + 3] = v.w;
        }
    }
    float acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.0f;
    float zacc = 0.0f, lloc = 0.0f, mrun = -INFINITY;

    if constexpr (EXACT) {
        for (int bs = 0; bs < nlist; bs += NB) {
            const int nb = min(NB, nlist - bs);
            const int nu = (nb + 15) >> 4;  // value rounds of this batch (uniform)
            // ---- round 2: the batch's key and value records (entries past nb re-read the last)
            uint32_t sl[VU + 1];
    #pragma unroll
            for (int u = 0; u <= VU; ++u) {
                const uint32_t t = (uint32_t)(t0 + list[bs + min(u < VU ? eg + 16 * u : lane, nb - 1)]);
                sl[u] = pbase[(t >> logP) - p0] + (t & tmask);
            }
            uint4 kb;
            uint32_t nc;
            if constexpr (!EXACT) load_key_t<KW>(p.c, sl[VU], kb, nc);
            uint4 kx[EXACT ? VU : 1][4];  // exact scores: binary16 key dims 32 q4 .. 32 q4 + 31
            if constexpr (EXACT) {
    #pragma unroll
                for (int u = 0; u < VU; ++u) {
                    if (u < nu) {
                        const uint4 *kr = reinterpret_cast<const uint4 *>(p.c.kf16 + (size_t)sl[u] * kD + 32 * q4);
    #pragma unroll
                        for (int k = 0; k < 4; ++k) kx[u][k] = kr[k];
                    }
                }
            }
            uint4 cw[VU];
            uint32_t szw[VU];
    #pragma unroll
            for (int u = 0; u < VU; ++u) {
                if (u < nu) {
                    const uint8_t *vr = val_rec(p.c, sl[u]);
                    __builtin_memcpy(&cw[u], vr + 16 * q4, 16);  // 8-byte aligned when Gv = 64
                    szw[u] = *reinterpret_cast<const uint32_t *>(vr + kD / 2 + 4 * grp);
                }
            }
            float s;
            float sx[EXACT ? VU : 1];  // exact scores of entries eg + 16 u (in all 4 lanes of the group)
            if constexpr (EXACT) {
                s = -INFINITY;
    #pragma unroll
                for (int u = 0; u < VU; ++u) {
                    sx[u] = -INFINITY;
                    if (u < nu) {
                        float a = 0.0f;
    #pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t w4[4] = {kx[u][k].x, kx[u][k].y, kx[u][k].z, kx[u][k].w};
    #pragma unroll
                            for (int e = 0; e < 8; ++e)
                                a = fmaf(qx[8 * k + e], half_bits_to_float((w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), a);
                        }
                        a = quad_sum(a);
                        sx[u] = eg + 16 * u < nb ? a : -INFINITY;
                    }
                    s = fmaxf(s, sx[u]);
                }
            } else {
                int A;
                score_key<1>(kb, nc, qs, &s, &A, 32 * KW);
                if (lane >= nb) s = -INFINITY;
            }
            const float mnew = fmaxf(mrun, wave_max(s));
            const float scale = (mrun == -INFINITY) ? 0.0f : exp2f((mrun - mnew) * p.klog);
            if (scale != 1.0f) {
                zacc *= scale;
                lloc *= scale;
    #pragma unroll
                for (int j = 0; j < 32; ++j) acc[j] *= scale;
            }
            mrun = mnew;
            float wx[EXACT ? VU : 1];
            if constexpr (EXACT) {
    #pragma unroll
                for (int u = 0; u < VU; ++u) {
                    wx[u] = (sx[u] == -INFINITY) ? 0.0f : exp2f((sx[u] - mnew) * p.klog);
                    if (q4 == 0) lloc += wx[u];  // each entry once
                }
            } else {
                const float w = (s == -INFINITY) ? 0.0f : exp2f((s - mnew) * p.klog);
                lloc += w;
                wbuf[lane] = w;
                wave_lds_sync();
            }
    #pragma unroll
            for (int u = 0; u < VU; ++u) {
                if (u < nu) {
                    float we;  // 0 past nb
                    if constexpr (EXACT) we = wx[u];
                    else we = wbuf[eg + 16 * u];
                    const float sf = half_bits_to_float(szw[u] & 0xFFFFu);
                    const float zf = half_bits_to_float(szw[u] >> 16);
                    const float ws = we * sf * kCodeUnscale;  // exact: by 2^9
                    zacc = fmaf(we, zf, zacc);
                    const uint32_t cwk[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
    #pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        // word k holds dims 32 q4 + 8k .. + 7
                        float c[8];
                        unpack_codes_e4m3(cwk[k], c);  // c * 2^-9
    #pragma unroll
                        for (int j = 0; j < 8; ++j) acc[8 * k + j] = fmaf(ws, c[j], acc[8 * k + j]);
                    }
                }
            }
            if constexpr (!EXACT) wave_lds_sync();  // wbuf is rewritten by the next batch
        }
    } else {
        // Proxy scores: the batches are software-pipelined in two register sets, the next
        // batch's key and value gathers in flight while this batch is scored and summed (a
        // dense head's wave works through many batches, each otherwise paying a full gather
        // latency).  Value rounds past the batch's entries re-read its last entry and are
        // not summed.
        struct Gather {
            uint4 kb;
            uint32_t nc;
            uint4 cw[VU];
            uint32_t szw[VU];
        };
        auto gather = [&](int bs, Gather &G) {
            const int nb = min(NB, nlist - bs);
            uint32_t sl[VU + 1];
#pragma unroll
            for (int u = 0; u <= VU; ++u) {
                const uint32_t t = (uint32_t)(t0 + list[bs + min(u < VU ? eg + 16 * u : lane, nb - 1)]);
                sl[u] = pbase[(t >> logP) - p0] + (t & tmask);
            }
            load_key_t<KW>(p.c, sl[VU], G.kb, G.nc);
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                const uint8_t *vr = val_rec(p.c, sl[u]);
                __builtin_memcpy(&G.cw[u], vr + 16 * q4, 16);  // 8-byte aligned when Gv = 64
                G.szw[u] = *reinterpret_cast<const uint32_t *>(vr + kD / 2 + 4 * grp);
            }
        };
        auto attend = [&](int bs, const Gather &G) {
            const int nb = min(NB, nlist - bs);
            const int nu = (nb + 15) >> 4;  // value rounds of this batch (uniform)
            float s;
            int A;
            score_key<1>(G.kb, G.nc, qs, &s, &A, 32 * KW);
            if (lane >= nb) s = -INFINITY;
            const float mnew = fmaxf(mrun, wave_max(s));
            const float scale = (mrun == -INFINITY) ? 0.0f : exp2f((mrun - mnew) * p.klog);
            if (scale != 1.0f) {
                zacc *= scale;
                lloc *= scale;
#pragma unroll
                for (int j = 0; j < 32; ++j) acc[j] *= scale;
            }
            mrun = mnew;
            const float w = (s == -INFINITY) ? 0.0f : exp2f((s - mnew) * p.klog);
            lloc += w;
            wbuf[lane] = w;
            wave_lds_sync();
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                if (u < nu) {
                    const float we = wbuf[eg + 16 * u];  // 0 past nb
                    const float sf = half_bits_to_float(G.szw[u] & 0xFFFFu);
                    const float zf = half_bits_to_float(G.szw[u] >> 16);
                    const float ws = we * sf * kCodeUnscale;  // exact: by 2^9
                    zacc = fmaf(we, zf, zacc);
                    const uint32_t cwk[4] = {G.cw[u].x, G.cw[u].y, G.cw[u].z, G.cw[u].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        // word k holds dims 32 q4 + 8k .. + 7
                        float c[8];
                        unpack_codes_e4m3(cwk[k], c);  // c * 2^-9
#pragma unroll
                        for (int j = 0; j < 8; ++j) acc[8 * k + j] = fmaf(ws, c[j], acc[8 * k + j]);
                    }
                }
            }
            wave_lds_sync();  // wbuf is rewritten by the next batch
        };
        Gather ga, gb;
        if (nlist > 0) gather(0, ga);
        for (int bs = 0; bs < nlist; bs += 2 * NB) {
            if (bs + NB < nlist) gather(bs + NB, gb);
            attend(bs, ga);
            if (bs + NB >= nlist) break;
            if (bs + 2 * NB < nlist) gather(bs + 2 * NB, ga);
            attend(bs + NB, gb);
        }
    }

    // ---- weight sum, then the value sums over the 16 entry groups: the 4 groups of a
    // 16-lane row by DPP rotations, the 4 rows through LDS (the list's slice, which the
    // fence below keeps from being overwritten before the last batch has read it)
    const float lsum = wave_sum(lloc);
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        acc[j] += dpp_ror(acc[j], 4);
        acc[j] += dpp_ror(acc[j], 8);
    }
    zacc += dpp_ror(zacc, 4);
    zacc += dpp_ror(zacc, 8);
    if ((lane & 15) < 4) {
        float4 *dst = red[lane >> 4][q4];
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = make_float4(acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]);
        dst[8].x = zacc;
    }
    wave_lds_sync();
    const size_t pidx = bh * g.NCA + c0;
    {
        // lane l: dims 2l, 2l + 1 (dim block l / 16, float4 (l & 15) / 2, half l & 1)
        const int qb = lane >> 4, f4 = (lane & 15) >> 1, hf = lane & 1;
        float v0 = 0.0f, v1 = 0.0f, z = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 a = red[r][qb][f4];
            v0 += hf ? a.z : a.x;
            v1 += hf ? a.w : a.y;
            z += red[r][qb][8].x;
        }
        reinterpret_cast<float2 *>(p.po + pidx * kD)[lane] = make_float2(v0 + z, v1 + z);
    }
    if (lane == 0) {
        p.pm[pidx] = mrun;
        p.pl[pidx] = lsum;
    } else if (lane < span && c0 + lane < g.NCA) {
        p.pm[pidx + lane] = -INFINITY;  // the span's other chunks: empty partials
        p.pl[pidx + lane] = 0.0f;
    }
}

// ---------------------------------------------------------------------------------------
// Attention mass of the tail tokens and the high-precision tier, once the query head's
// softmax is known (max score M, weight sum D): every such token adds its weight
// exp2((s - M) log2e / sqrt(D)) / D to its mass, with its exact score s recomputed by a
// group of 16 lanes (8 dims each, so the rounding may differ from the tail pass in the last
// bits); the query heads of a KV head add atomically.  The first round's loads (query,
// center, key words, entry positions) are issued when the merge starts, so that they are
// done by the time M and D are.
// ---------------------------------------------------------------------------------------
constexpr int kMassNU = 4;  // tokens per 16-lane group and round

struct MassPrefetch {
    float qx[8], cx[8];
    uint4 kw[kMassNU];
    bool ok[kMassNU];
    int nt, ntot;
};

__device__ __forceinline__ const uint16_t *mass_key(const MassParams &p, int b, int kvh, int Hkv, int nt, int j)
{
    return j < nt ? p.tk + (((size_t)b * p.tcap + j) * Hkv + kvh) * kD
                  : p.hk + (((size_t)b * Hkv + kvh) * p.hcap + (j - nt)) * kD;
}

__device__ __forceinline__ void mass_round_load(const MassParams &p, int b, int kvh, int Hkv, int j0, MassPrefetch &f)
{
    const int tid = threadIdx.x, step = (int)blockDim.x >> 4, sub = tid & 15;
#pragma unroll
    for (int u = 0; u < kMassNU; ++u) {
        const int j = j0 + u * step + (tid >> 4);
        f.ok[u] = j < f.ntot && (j < f.nt || p.hpos[((size_t)b * Hkv + kvh) * p.hcap + (j - f.nt)] >= 0);
        f.kw[u] = j < f.ntot ? reinterpret_cast<const uint4 *>(mass_key(p, b, kvh, Hkv, f.nt, j))[sub]
                             : make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void mass_prefetch(const MassParams &p, int b, int h, int G, int Hkv, MassPrefetch &f)
{
    const int kvh = h / G, sub = threadIdx.x & 15;
    const size_t bh = (size_t)b * (G * Hkv) + h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        f.qx[e] = p.q[bh * kD + 8 * sub + e];  // q is only 4-byte aligned
        f.cx[e] = p.center ? p.center[(size_t)kvh * kD + 8 * sub + e] : 0.0f;
    }
    f.nt = p.tk ? min(max(p.tlen[b], 0), p.tcap) : 0;
    f.ntot = f.nt + (p.hk ? p.hcap : 0);
    mass_round_load(p, b, kvh, Hkv, 0, f);
}

__device__ __forceinline__ void mass_finish(const MassParams &p, int b, int h, int G, int Hkv, float M, float D,
                                            float klog, MassPrefetch &f)
{
    const int kvh = h / G, tid = threadIdx.x, sub = tid & 15, step = (int)blockDim.x >> 4;
    // <q, c>: the 16-lane group's own sum over the 128 dims
    float qc = 0.0f;
    if (p.center) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qc = fmaf(f.qx[e], f.cx[e], qc);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) qc += __shfl_xor(qc, o);
    }
    const float inv = D > 0.0f ? 1.0f / D : 0.0f;
    for (int j0 = 0; j0 < f.ntot; j0 += kMassNU * step) {  // the same trip count for every lane
        if (j0 > 0) mass_round_load(p, b, kvh, Hkv, j0, f);
#pragma unroll
        for (int u = 0; u < kMassNU; ++u) {
            const int j = j0 + u * step + (tid >> 4);
            const uint32_t w[4] = {f.kw[u].x, f.kw[u].y, f.kw[u].z, f.kw[u].w};
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaf(f.qx[e], half_bits_to_float((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), a);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o);
            if (f.ok[u] && sub == 0 && D > 0.0f) {
                float *dst = j < f.nt ? p.tmass + ((size_t)b * p.tcap + j) * Hkv + kvh
                                      : p.hmass + ((size_t)b * Hkv + kvh) * p.hcap + (j - f.nt);
                atomicAdd(dst, exp2f((a - qc - M) * klog) * inv);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Split-K merge, one 1024-thread block per (query head, sequence):
//   out = sum_c a_c o_c / sum_c a_c l_c,  a_c = exp2((m_c - M) log2e/sqrt(D)),  M = max m_c.
// Thread (d, slice) sums the chunks c = slice (mod 8) for dim d; a chunk of zero weight (no
// attended token, or an empty partial of a Top-p span) adds nothing, and its value sums are
// not read.  The value sums of the
// first 8 PF chunks are loaded first, so that their reads overlap the max and weight
// reductions.
// ---------------------------------------------------------------------------------------
// PF: chunks per thread loaded ahead, no more than the plan's NCA chunks give a thread (8
// slices), so that no load is spent on a slot past the last; fewer beside the mass prefetch.
template <bool MASS, int PF>
__global__ __launch_bounds__(1024) void k_merge(MergeParams p)
{
    constexpr int kT = 1024, NS = kT / kD;  // threads, chunk slices
    __shared__ float alpha[kMaxChunks];
    __shared__ float redf[2][kT / 64];
    __shared__ float part[NS][kD];
    const DecodeGeom &g = p.g;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = (size_t)b * g.Hq + h;
    const int L = g.seq_lens[b];
    const int CHa = g.CH * g.KA;
    const int nch = L > 0 ? (L + CHa - 1) / CHa : 0;
    const int d = tid & (kD - 1), sl = tid >> 7;
    MassPrefetch mf;
    if (MASS) mass_prefetch(p.mass, b, h, g.Hq / g.Hkv, g.Hkv, mf);
    // Loads and sums below are branch-free (so that a round's loads are all in flight at
    // once): a chunk past the end, or one without weight, re-reads chunk 0 and is not added.
    const float *po = p.po + bh * g.NCA * kD + d;
    float v[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int c = sl + NS * i;
        v[i] = po[(size_t)(c < nch ? c : 0) * kD];
    }
    // the first kT chunks' max and weight sum are read once, with the value sums in flight
    const float mc0 = tid < nch ? p.pm[bh * g.NCA + tid] : -INFINITY;
    const float lc0 = tid < nch ? p.pl[bh * g.NCA + tid] : 0.0f;
    float m = mc0;
    for (int c = tid + kT; c < nch; c += kT) m = fmaxf(m, p.pm[bh * g.NCA + c]);
    m = wave_max(m);
    if (lane == 0) redf[0][wave] = m;
    __syncthreads();
    const float tm = p.tm ? p.tm[bh] : -INFINITY;  // the binary16 tail's partial, if any
    float M = fmaxf(redf[0][0], tm);
#pragma unroll
    for (int w = 1; w < kT / 64; ++w) M = fmaxf(M, redf[0][w]);
    const float at = (tm == -INFINITY) ? 0.0f : exp2f((tm - M) * p.klog);
    float den = 0.0f;
    if (tid < nch) {
        const float a = (mc0 == -INFINITY) ? 0.0f : exp2f((mc0 - M) * p.klog);
        alpha[tid] = a;
        den = a * lc0;
    }
    for (int c = tid + kT; c < nch; c += kT) {
        const float mc = p.pm[bh * g.NCA + c];
        const float a = (mc == -INFINITY) ? 0.0f : exp2f((mc - M) * p.klog);
        alpha[c] = a;
        den = fmaf(a, p.pl[bh * g.NCA + c], den);
    }
    den = wave_sum(den);
    if (lane == 0) redf[1][wave] = den;
    __syncthreads();  // also publishes alpha
    float D = (at != 0.0f) ? at * p.tl[bh] : 0.0f;
#pragma unroll
    for (int w = 0; w < kT / 64; ++w) D += redf[1][w];
    float num = 0.0f;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const int c = sl + NS * i;
        const float a = alpha[c < nch ? c : 0];
        num = (c < nch && a != 0.0f) ? fmaf(a, v[i], num) : num;
    }
    for (int c0 = sl + NS * PF; c0 < nch; c0 += NS * PF) {
        // the rest in rounds of PF loads in flight; the weights are known by now, so empty
        // partials (chunks that a wave covering several wrote as such) are not fetched
        float a[PF];
        bool any = false;
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int c = c0 + NS * i;
            a[i] = c < nch ? alpha[c] : 0.0f;
            any |= a[i] != 0.0f;
        }
        if (!__any(any)) continue;  // wave-uniform: a round of empty partials only
#pragma unroll
        for (int i = 0; i < PF; ++i) v[i] = po[(size_t)(a[i] != 0.0f ? c0 + NS * i : 0) * kD];
#pragma unroll
        for (int i = 0; i < PF; ++i) num = a[i] != 0.0f ? fmaf(a[i], v[i], num) : num;
    }
    part[sl][d] = num;
    __syncthreads();
    if (tid < kD) {
        float t = (at != 0.0f) ? at * p.to[bh * kD + d] : 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) t += part[s2][d];
        p.out[bh * kD + d] = D > 0.0f ? t / D : 0.0f;
    }
    if (MASS) mass_finish(p.mass, b, h, g.Hq / g.Hkv, g.Hkv, M, D, p.klog, mf);
}

// ---------------------------------------------------------------------------------------
// Argument checker (KV_DEBUG=1): block b checks sequence b's token range and the page table
// entries that cover it; every read stays inside seq_lens / start_pos [B] and the B x
// max_pages table, so a bad entry is reported instead of dereferenced.  The first failing
// thread (atomicCAS on the code word) records (code, b, page index or -1, value).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_check_clear(int32_t *flag)
{
    if (threadIdx.x < 4) flag[threadIdx.x] = 0;
}

__device__ __forceinline__ void check_fail(int32_t *flag, int code, int b, int j, int v)
{
    if (atomicCAS(&flag[0], 0, code) == 0) {
        flag[1] = b;
        flag[2] = j;
        flag[3] = v;
    }
}

__global__ __launch_bounds__(256) void k_check(CheckParams p, int32_t *flag)
{
    const int b = blockIdx.x;
    long lo = 0, hi = 0;  // token range [lo, hi)
    if (p.seq_lens) {
        const int L = p.seq_lens[b];
        if (L < 0 || L > p.max_seq_len) {
            if (threadIdx.x == 0) check_fail(flag, kCheckLen, b, -1, L);
            return;
        }
        hi = L;
    } else {
        const int sp = p.start_pos[b];
        if (sp < 0 || (long)sp + p.n_new > ((long)p.max_pages << p.logP)) {
            if (threadIdx.x == 0) check_fail(flag, kCheckStart, b, -1, sp);
            return;
        }
        lo = sp;
        hi = (long)sp + p.n_new;
    }
    if (hi <= lo) return;
    const long j0 = lo >> p.logP, j1 = (hi - 1) >> p.logP;  // j1 < max_pages by the checks above
    for (long j = j0 + threadIdx.x; j <= j1; j += blockDim.x) {
        const int id = p.page_table[(size_t)b * p.max_pages + j];
        if (id < 0 || id >= p.num_pages) check_fail(flag, kCheckPage, b, (int)j, id);
    }
}

// The full-softmax kernel for the cache's key record width.  The matrix-core form when its
// A operand has at least 4 rows in use (heads x value groups); one head over 64-dim groups
// (2 rows) stays on the vector units, which measured faster there.
template <int GB, int GV>
void launch_full(const AttendParams &p, dim3 grid, hipStream_t s)
{
    const bool big = p.c.logP >= 6;
    if constexpr (GB * (kD / GV) < 4) {
        if (p.c.kw == 4) {
            if (big) KVC_LAUNCH((k_attend_full<GB, GV, 4, true>), grid, dim3(64), s, p);
            else KVC_LAUNCH((k_attend_full<GB, GV, 4, false>), grid, dim3(64), s, p);
        } else {
            if (big) KVC_LAUNCH((k_attend_full<GB, GV, 2, true>), grid, dim3(64), s, p);
            else KVC_LAUNCH((k_attend_full<GB, GV, 2, false>), grid, dim3(64), s, p);
        }
    } else {
        if (p.c.kw == 4) {
            if (big) KVC_LAUNCH((k_attend_full_mf<GB, GV, 4, true>), grid, dim3(64), s, p);
            else KVC_LAUNCH((k_attend_full_mf<GB, GV, 4, false>), grid, dim3(64), s, p);
        } else {
            if (big) KVC_LAUNCH((k_attend_full_mf<GB, GV, 2, true>), grid, dim3(64), s, p);
            else KVC_LAUNCH((k_attend_full_mf<GB, GV, 2, false>), grid, dim3(64), s, p);
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_qprep(const QprepParams &p, hipStream_t s)
{
    const float isd = (float)(1.0 / sqrt((double)kD));
    const long blocks = (long)p.BH * (p.has_tail ? 2 : 1) + p.app_blocks;
    const bool wide = p.has_tail || p.app_blocks > 0;
    const dim3 grid((unsigned)blocks), blk(wide ? 256 : 128);
    if (p.has_tail) KVC_LAUNCH(k_qprep<1>, grid, blk, s, p, isd);
    else if (p.app_blocks > 0 && p.app.rot_kind == 1) KVC_LAUNCH(k_qprep<2>, grid, blk, s, p, isd);
    else if (p.app_blocks > 0) KVC_LAUNCH(k_qprep<3>, grid, blk, s, p, isd);
    else KVC_LAUNCH(k_qprep<0>, grid, blk, s, p, isd);
    return hipGetLastError();
}

hipError_t launch_score(const ScoreParams &p, hipStream_t s)
{
    const dim3 grid(p.g.NC, p.g.Hkv * p.g.nsub, p.g.B);
    const dim3 blk(64);
    const bool dbg = p.dbg_scores || p.dbg_iscores;
    if (!dbg && p.dl && p.g.CH == kTopPChunk) {
        switch (p.g.GB) {
        case 1:
            if (p.c.kw == 4) KVC_LAUNCH((k_score_topp<1, 4>), grid, blk, s, p);
            else KVC_LAUNCH((k_score_topp<1, 2>), grid, blk, s, p);
            break;
        case 2:
            if (p.c.kw == 4) KVC_LAUNCH((k_score_topp<2, 4>), grid, blk, s, p);
            else KVC_LAUNCH((k_score_topp<2, 2>), grid, blk, s, p);
            break;
        default:
            if (p.c.kw == 4) KVC_LAUNCH(k_score_topp_mf<4>, grid, blk, s, p);
            else KVC_LAUNCH(k_score_topp_mf<2>, grid, blk, s, p);
            break;
        }
    } else {
        // debug scores: the Top-p chunks, or the larger chunks of a full-softmax decode
        switch (p.g.GB) {
        case 1: KVC_LAUNCH((k_score<1, true, 8192>), grid, blk, s, p); break;
        case 2: KVC_LAUNCH((k_score<2, true, 4096>), grid, blk, s, p); break;
        default: KVC_LAUNCH((k_score<4, true, 2048>), grid, blk, s, p); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_bin_scores(const BinScoresParams &p, hipStream_t s)
{
    KVC_LAUNCH(k_bin_scores, dim3(p.g.NC, p.g.Hq, p.g.B), dim3(kBlock), s, p);
    return hipGetLastError();
}

hipError_t launch_hist(const HistParams &p, hipStream_t s)
{
    if (p.fused) {
        KVC_LAUNCH(k_hist_thresh, dim3(p.g.Hq, p.g.B), dim3(kHistThreads), s, p);
        return hipGetLastError();
    }
    KVC_LAUNCH(k_hist, dim3(p.nsplit, p.g.Hq, p.g.B), dim3(kHistThreads), s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KVC_LAUNCH(k_thresh, dim3(p.g.Hq, p.g.B), dim3(1024), s, p);
    return hipGetLastError();
}

hipError_t launch_select(const SelectParams &p, hipStream_t s)
{
    const dim3 grid(p.g.NC, p.g.Hq, p.g.B);
    KVC_LAUNCH(k_sel_count, grid, dim3(kBlock), s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    KVC_LAUNCH(k_sel_write, grid, dim3(kBlock), s, p);
    return hipGetLastError();
}

hipError_t launch_attend(const AttendParams &p, bool select, hipStream_t s)
{
    if (select) {
        // blocks of kAttendWaves waves per (kAttendWaves attention chunks, dispatch rank)
        const dim3 grid((p.g.NCA + kAttendWaves - 1) / kAttendWaves, p.g.Hq, p.g.B);
        if (p.g.CH * p.g.KA != kTopPAttendChunk) return hipErrorInvalidValue;
        const bool w4 = p.c.kw == 4;
        const dim3 blk(64 * kAttendWaves);
        if (p.c.kf16) {
            if (w4) KVC_LAUNCH((k_attend_topp<true, 4, 0>), grid, blk, s, p);
            else KVC_LAUNCH((k_attend_topp<true, 2, 0>), grid, blk, s, p);
        } else if (p.g.GB == 4 && p.c.logP >= 6) {
            // groups of 4 heads over pages of >= 64 tokens: with the masked chunk pass
            if (p.c.Gv == 32) {
                if (w4) KVC_LAUNCH((k_attend_topp<false, 4, 32>), grid, blk, s, p);
                else KVC_LAUNCH((k_attend_topp<false, 2, 32>), grid, blk, s, p);
            } else {
                if (w4) KVC_LAUNCH((k_attend_topp<false, 4, 64>), grid, blk, s, p);
                else KVC_LAUNCH((k_attend_topp<false, 2, 64>), grid, blk, s, p);
            }
        } else {
            if (w4) KVC_LAUNCH((k_attend_topp<false, 4, 0>), grid, blk, s, p);
            else KVC_LAUNCH((k_attend_topp<false, 2, 0>), grid, blk, s, p);
        }
    } else {
        // one wave per (chunk, KV-head group, sequence)
        const dim3 grid(p.g.NCA, p.g.Hkv * p.g.nsub, p.g.B);
        if (p.g.CH > kMaxFullChunk || p.g.KA != 1) return hipErrorInvalidValue;
        const bool g32 = p.c.Gv == 32;
        switch (p.g.GB) {
        case 1:
            if (g32) launch_full<1, 32>(p, grid, s);
            else launch_full<1, 64>(p, grid, s);
            break;
        case 2:
            if (g32) launch_full<2, 32>(p, grid, s);
            else launch_full<2, 64>(p, grid, s);
            break;
        default:
            if (g32) launch_full<4, 32>(p, grid, s);
            else launch_full<4, 64>(p, grid, s);
            break;
        }
    }
    return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];  // the device address of each device's copy of `scratch`
}  // namespace

hipError_t static_scratch(hipStream_t s, void **ptr)
{
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (s) {
        e = hipStreamGetDevice(s, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        // once per device, with that device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_check(const CheckParams &p, int32_t *flag_host, hipStream_t s)
{
    int32_t *flag = nullptr;  // this device's copy of the flag
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&flag), HIP_SYMBOL(g_check_flag));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_check_clear, dim3(1), dim3(64), 0, s, flag);
    hipLaunchKernelGGL(k_check, dim3(p.B), dim3(256), 0, s, p, flag);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(flag_host, flag, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, s);
}

hipError_t launch_merge(const MergeParams &p, hipStream_t s)
{
    const dim3 grid(p.g.Hq, p.g.B);
    // chunks per thread (8 slices of 128 dims); up to 16 of them, 8 loaded ahead and the rest
    // after the weights are known (Top-p partials of spans are often empty and then skipped)
    const int per = (p.g.NCA + 7) / 8;
    if (p.has_mass) {
        if (per <= 16) KVC_LAUNCH((k_merge<true, 8>), grid, dim3(1024), s, p);
        else KVC_LAUNCH((k_merge<true, 16>), grid, dim3(1024), s, p);
    } else {
        if (per <= 16) KVC_LAUNCH((k_merge<false, 8>), grid, dim3(1024), s, p);
        else if (per <= 32) KVC_LAUNCH((k_merge<false, 16>), grid, dim3(1024), s, p);
        else KVC_LAUNCH((k_merge<false, 32>), grid, dim3(1024), s, p);
    }
    return hipGetLastError();
}

}  // namespace kvc
