// Decode kernels: query preparation, binary x INT4 proxy scores, adaptive Top-p (bin
// distances, histogram, threshold, ordered selection), chunked attention over the 4-bit
// values, and the split-K merge.
//
// Method: "RaBitQCache" (abstract and key design: int4 query, binary x INT4 proxy score,
// adaptive Top-p) and "H1B-KV" (technical framework: attention weights from the 1-bit key
// sketch, output from the 4-bit values).
//
// Work decomposition.  A sequence is cut into chunks of CH tokens (CH a power of two,
// 256..8192).  One 256-thread block works on one (chunk, KV head, sequence) and on GB <= 4
// of the query heads that share the KV head (GQA), so every key word and value byte it
// streams from HBM serves all GB heads.  Partial results (max score, weight sum, weighted
// value sum) of all chunks are merged per (sequence, query head) at the end.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

// First query head of block (hb = kv head * nsub + sub) and its KV head.
__device__ __forceinline__ void block_heads(const DecodeGeom &g, int hb, int &kvh, int &hq0)
{
    kvh = hb / g.nsub;
    const int sub = hb - kvh * g.nsub;
    hq0 = kvh * g.G + sub * g.GB;
}

__device__ __forceinline__ size_t token_slot(const DecodeGeom &g, const CacheView &c, int b, int kvh,
                                             int t)
{
    const int page = g.page_table[(size_t)b * g.max_pages + (t >> c.logP)];
    return ((size_t)page * c.Hkv + kvh) * c.P + (t & (c.P - 1));
}

// Block-wide max of GB ints per thread (256 threads); result broadcast through LDS.
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
// Query preparation (one 128-thread block per (sequence, query head), one thread per dim):
//   dense:    q'_r = fmaf chain over j ascending of R[r][j] * q_j (binary32)
//   hadamard: x = sigma * q, in-place fast Walsh-Hadamard butterflies h = 1..64 (binary32),
//             q' = x * fp32(1/sqrt(D))
//   v_l = min q', delta = (max q' - v_l) / 15, u = clamp(rint((q' - v_l) / delta), 0, 15)
//   (u = 0 when delta == 0); bit-planes of u; c0 = v_l/sqrt(D), c1 = delta/sqrt(D).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_qprep(QprepParams p, float isd)
{
    __shared__ float xs[kD];
    __shared__ float redf[4];
    __shared__ int redi[2];
    const int bh = blockIdx.x, r = threadIdx.x;
    const int lane = r & 63, wave = r >> 6;
    const float *q = p.q + (size_t)bh * kD;
    float x;
    if (p.rot_kind == 0) {
        xs[r] = q[r];
        __syncthreads();
        const uint4 *Rr = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(p.rot) + r * kD);
        float a = 0.0f;
        for (int c = 0; c < kD / 8; ++c) {
            const uint4 raw = Rr[c];
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
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
    // min / max over the 128 rotated coordinates
    float mn = x, mx = x;
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
    if (delta != 0.0f) {
        float t = rintf((x - vl) / delta);
        t = fminf(fmaxf(t, 0.0f), 15.0f);
        u = (int)t;
    }
    int su = wave_sum_i(u);
    if (lane == 0) redi[wave] = su;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t m = __ballot((u >> j) & 1);
        if (lane == 0) {
            p.qpl[(size_t)bh * 16 + j * 4 + 2 * wave] = (uint32_t)m;
            p.qpl[(size_t)bh * 16 + j * 4 + 2 * wave + 1] = (uint32_t)(m >> 32);
        }
    }
    __syncthreads();
    su = redi[0] + redi[1];
    if (r == 0) p.qpar[bh] = make_float4(vl * isd, delta * isd, __int_as_float(su), 0.0f);
    if (p.dbg_codes) p.dbg_codes[(size_t)bh * kD + r] = (uint8_t)u;
    if (r == 0 && p.dbg_params) {
        p.dbg_params[bh * 4 + 0] = vl;
        p.dbg_params[bh * 4 + 1] = delta;
        p.dbg_params[bh * 4 + 2] = vl * isd;
        p.dbg_params[bh * 4 + 3] = delta * isd;
    }
    if (r == 0 && p.dbg_sumu) p.dbg_sumu[bh] = su;
}

// ---------------------------------------------------------------------------------------
// Score pass (Top-p first pass, and debug scores): per (chunk, KV head, sequence) block,
// the proxy score of every token of the chunk for GB query heads.  Writes the bin distance
// to the chunk's top bin (uint16, saturated at 8192: no token that far below a chunk's top
// can be selected, since the threshold distance is < 8192) and the chunk's top bin.
// ---------------------------------------------------------------------------------------
template <int GB>
__global__ __launch_bounds__(256) void k_score(ScoreParams p)
{
    __shared__ int ebuf[8192];
    __shared__ int red[4 * GB];
    __shared__ int emax_s[GB];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int bh0 = b * g.Hq + hq0;
    QueryState<GB> qs;
    load_query<GB>(qs, p.qpl, p.qpar, bh0);
    int lm[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) lm[h] = -kBinClamp;
    const uint4 *kb4 = reinterpret_cast<const uint4 *>(p.c.key_bits);
    for (int tl = threadIdx.x; tl < n; tl += kBlock) {
        const int t = t0 + tl;
        const size_t slot = token_slot(g, p.c, b, kvh, t);
        const uint4 kb = kb4[slot];
        const uint32_t nc = p.c.key_nc[slot];
        float s[GB];
        int A[GB];
        score_key<GB>(kb, nc, qs, s, A);
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const int e = score_bin(s[h], p.kbin);
            ebuf[h * g.CH + tl] = e;
            lm[h] = max(lm[h], e);
            if (p.dbg_scores) p.dbg_scores[(size_t)(bh0 + h) * g.ld + t] = s[h];
            if (p.dbg_iscores) p.dbg_iscores[(size_t)(bh0 + h) * g.ld + t] = A[h];
        }
    }
    if (!p.dl) return;
    block_reduce<GB>(lm, red, emax_s, MaxI());
    if (threadIdx.x < GB) p.lmax[(size_t)(bh0 + threadIdx.x) * g.NC + chunk] = emax_s[threadIdx.x];
    for (int tl = threadIdx.x; tl < n; tl += kBlock) {
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const int d = emax_s[h] - ebuf[h * g.CH + tl];
            p.dl[(size_t)(bh0 + h) * g.Lpad + t0 + tl] = (uint16_t)min(d, kBins);
        }
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

// Top bin of (b, h): max over the chunk top bins.
__device__ __forceinline__ int global_top_bin(const DecodeGeom &g, const int32_t *lmax, size_t bh,
                                              int nch, int *red /* [4] */, int *out /* [1] */)
{
    int m[1] = {-kBinClamp};
    for (int c = threadIdx.x; c < nch; c += kBlock) m[0] = max(m[0], lmax[bh * g.NC + c]);
    block_reduce<1>(m, red, out, MaxI());
    return out[0];
}

// ---------------------------------------------------------------------------------------
// Histogram pass: per (split, query head, sequence) block, counts of tokens per bin
// distance d = (e_max - chunk top) + distance-to-chunk-top, for d < 8192.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_hist(HistParams p)
{
    __shared__ uint32_t hist[kBins];
    __shared__ int delta[1024];
    __shared__ int red[4];
    __shared__ int top[1];
    const DecodeGeom &g = p.g;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t bh = (size_t)b * g.Hq + h;
    const int L = g.seq_lens[b];
    const int nch = (L + g.CH - 1) >> g.logCH;
    for (int i = threadIdx.x; i < kBins; i += kBlock) hist[i] = 0u;
    const int emax = global_top_bin(g, p.lmax, bh, nch, red, top);
    const int c0 = split * p.cps;
    const int c1 = min(nch, c0 + p.cps);
    for (int c = c0 + (int)threadIdx.x; c < c1; c += kBlock) delta[c - c0] = emax - p.lmax[bh * g.NC + c];
    __syncthreads();
    if (c0 < c1) {
        const int tb = c0 << g.logCH;
        const int te = min(L, c1 << g.logCH);
        const uint16_t *row = p.dl + bh * g.Lpad;
        // 8 tokens per thread-iteration (tb is a multiple of CH >= 256, so 16-byte aligned)
        for (int t = tb + 8 * (int)threadIdx.x; t < te; t += 8 * kBlock) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(row + t);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tt = t + e;
                if (tt < te) {
                    const int dloc = (int)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                    const int d = delta[(tt >> g.logCH) - c0] + dloc;
                    if (d < kBins) atomicAdd(&hist[d], 1u);
                }
            }
        }
    }
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(p.hist + (bh * p.nsplit + split) * kBins);
    for (int i = threadIdx.x; i < kBins / 4; i += kBlock)
        dst[i] = make_uint4(hist[4 * i], hist[4 * i + 1], hist[4 * i + 2], hist[4 * i + 3]);
}

// ---------------------------------------------------------------------------------------
// Threshold: per (query head, sequence) block.  With W(d) = T[d mod 256] >> (d / 256),
// T[j] = round(2^(32 - j/256)):  Z = sum_d cnt[d] W(d),  T_p = ceil(Z * pfx / 2^24),
// b* = min { b : sum_{d <= b} cnt[d] W(d) >= T_p }, count = sum_{d <= b*} cnt[d].
// Thread t owns bins 32t .. 32t+31.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_threshold(ThresholdParams p)
{
    __shared__ uint64_t T[256];
    __shared__ uint64_t wsum[4];
    __shared__ int red[4];
    __shared__ int top[1];
    __shared__ int bstar_s;
    __shared__ int cnt_s[4];
    const DecodeGeom &g = p.g;
    const int h = blockIdx.x, b = blockIdx.y;
    const size_t bh = (size_t)b * g.Hq + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = g.seq_lens[b];
    T[tid] = (uint64_t)rint(ldexp(exp2(-(double)tid / 256.0), 32));
    const int nch = (L + g.CH - 1) >> g.logCH;
    const int emax = global_top_bin(g, p.lmax, bh, nch, red, top);  // includes barriers
    if (L <= 0) {
        if (tid == 0) {
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
    uint32_t cnt[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) cnt[k] = 0u;
    for (int s = 0; s < p.nsplit; ++s) {
        const uint4 *src = reinterpret_cast<const uint4 *>(p.hist + (bh * p.nsplit + s) * kBins + 32 * tid);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint4 v = src[k];
            cnt[4 * k] += v.x;
            cnt[4 * k + 1] += v.y;
            cnt[4 * k + 2] += v.z;
            cnt[4 * k + 3] += v.w;
        }
    }
    // d >> 8 is the same for all 32 bins of a thread
    const int shift = (32 * tid) >> 8;
    uint64_t mine = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) mine += (uint64_t)cnt[k] * (T[(32 * tid + k) & 255] >> shift);
    // exclusive prefix of the per-thread masses
    uint64_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint64_t before = incl - mine;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const uint64_t Z = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const uint64_t lo = Z * (uint64_t)p.pfx;
    uint64_t hi = __umul64hi(Z, (uint64_t)p.pfx);
    const uint64_t lo2 = lo + ((1ull << 24) - 1);
    hi += (lo2 < lo) ? 1 : 0;
    const uint64_t Tp = (hi << 40) | (lo2 >> 24);
    if (tid == 0) bstar_s = (Tp == 0) ? 0 : kBins - 1;
    __syncthreads();
    if (Tp > 0 && before < Tp && before + mine >= Tp) {
        uint64_t F = before;
        int bs = 32 * tid + 31;
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            F += (uint64_t)cnt[k] * (T[(32 * tid + k) & 255] >> shift);
            if (F >= Tp) {
                bs = 32 * tid + k;
                break;
            }
        }
        bstar_s = bs;
    }
    __syncthreads();
    const int bstar = bstar_s;
    int c = 0;
#pragma unroll
    for (int k = 0; k < 32; ++k)
        if (32 * tid + k <= bstar) c += (int)cnt[k];
    c = wave_sum_i(c);
    if (lane == 0) cnt_s[wave] = c;
    __syncthreads();
    if (tid == 0) {
        const int count = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
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

// Bin-distance threshold of a chunk: token kept when its distance to the chunk top bin is
// <= b* - (e_max - chunk top).
__device__ __forceinline__ int chunk_threshold(const int32_t *sel, const int32_t *lmax, size_t bh,
                                               int NC, int chunk)
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
// Attention over one chunk for GB query heads of one KV head.
//   SEL: tokens whose bin distance passes the head's Top-p threshold (Top-p decode);
//   otherwise every token of the chunk (full softmax).
// Phase 1 lists the chunk's tokens (SEL: ordered compaction of the kept ones), phase 2
// scores them (binary x INT4), phase 3 turns scores into weights exp2((s - m) log2e/sqrt(D))
// with the chunk max m, phase 4 accumulates weights x decoded 4-bit values (8 lanes per
// token, 16 dims per lane; the zero point is accumulated once per group), and the block
// writes (m, sum of weights, weighted sum) for the merge.
// ---------------------------------------------------------------------------------------
template <int GB, bool SEL>
__global__ __launch_bounds__(256) void k_attend(AttendParams p)
{
    __shared__ float wbuf[8192];               // scores, then weights: [entry][GB]
    __shared__ uint32_t list[SEL ? 4096 : 1];  // entry -> token offset | head mask << 16
    __shared__ float redf[4 * GB];
    __shared__ float mh[GB], lh[GB];
    __shared__ int wcnt[4];
    const DecodeGeom &g = p.g;
    const int chunk = blockIdx.x, b = blockIdx.z;
    int kvh, hq0;
    block_heads(g, blockIdx.y, kvh, hq0);
    const int L = g.seq_lens[b];
    const int t0 = chunk * g.CH;
    if (t0 >= L) return;
    const int n = min(g.CH, L - t0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh0 = (size_t)b * g.Hq + hq0;

    // ---- phase 1: entries
    int nlist = n;
    if (SEL) {
        int thr[GB];
#pragma unroll
        for (int h = 0; h < GB; ++h) thr[h] = chunk_threshold(p.sel, p.lmax, bh0 + h, g.NC, chunk);
        int base = 0;
        for (int tb = 0; tb < n; tb += kBlock) {
            const int tl = tb + tid;
            uint32_t mask = 0;
            if (tl < n) {
#pragma unroll
                for (int h = 0; h < GB; ++h)
                    if ((int)p.dl[(bh0 + h) * g.Lpad + t0 + tl] <= thr[h]) mask |= 1u << h;
            }
            const uint64_t m = __ballot(mask != 0);
            if (lane == 0) wcnt[wave] = __popcll(m);
            __syncthreads();
            int off = base;
            for (int w = 0; w < wave; ++w) off += wcnt[w];
            if (mask) list[off + __popcll(m & lanemask_lt())] = (uint32_t)tl | (mask << 16);
            base += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
            __syncthreads();
        }
        nlist = base;
    }

    // ---- phase 2: scores
    QueryState<GB> qs;
    load_query<GB>(qs, p.qpl, p.qpar, (int)bh0);
    float mloc[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) mloc[h] = -INFINITY;
    const uint4 *kb4 = reinterpret_cast<const uint4 *>(p.c.key_bits);
    for (int e = tid; e < nlist; e += kBlock) {
        int tl = e;
        uint32_t mask = (1u << GB) - 1u;
        if (SEL) {
            const uint32_t ent = list[e];
            tl = (int)(ent & 0xFFFFu);
            mask = ent >> 16;
        }
        const size_t slot = token_slot(g, p.c, b, kvh, t0 + tl);
        float s[GB];
        int A[GB];
        score_key<GB>(kb4[slot], p.c.key_nc[slot], qs, s, A);
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const float v = ((mask >> h) & 1u) ? s[h] : -INFINITY;
            wbuf[e * GB + h] = v;
            mloc[h] = fmaxf(mloc[h], v);
        }
    }
    block_reduce<GB>(mloc, redf, mh, MaxF());

    // ---- phase 3: weights
    float lloc[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) lloc[h] = 0.0f;
    for (int e = tid; e < nlist; e += kBlock) {
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const float v = wbuf[e * GB + h];
            const float w = (v == -INFINITY) ? 0.0f : exp2f((v - mh[h]) * p.klog);
            wbuf[e * GB + h] = w;
            lloc[h] += w;
        }
    }
    block_reduce<GB>(lloc, redf, lh, SumF());

    // ---- phase 4: weighted sum of decoded values (8 lanes per entry, 16 dims per lane)
    const int sub = lane & 7;        // dims 16*sub .. 16*sub+15
    const int eg = lane >> 3;        // entry within the wave-iteration
    float acc[GB][16];
    float zacc[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) {
        zacc[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[h][j] = 0.0f;
    }
    const int gv = p.c.Gv;
    const int grp = (16 * sub) / gv;
    const int ngrp = kD / gv;
    for (int e = wave * 8 + eg; e < nlist; e += 32) {
        const int tl = SEL ? (int)(list[e] & 0xFFFFu) : e;
        const size_t slot = token_slot(g, p.c, b, kvh, t0 + tl);
        const uint2 cw = *reinterpret_cast<const uint2 *>(p.c.val_codes + slot * (kD / 2) + 8 * sub);
        const uint32_t szw = p.c.val_sz[slot * ngrp + grp];
        const float sf = half_bits_to_float(szw & 0xFFFFu);
        const float zf = half_bits_to_float(szw >> 16);
        float c[16];
        const uint32_t lo0 = cw.x & 0x0F0F0F0Fu, hi0 = (cw.x >> 4) & 0x0F0F0F0Fu;
        const uint32_t lo1 = cw.y & 0x0F0F0F0Fu, hi1 = (cw.y >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            c[2 * m] = (float)((lo0 >> (8 * m)) & 0xFFu);
            c[2 * m + 1] = (float)((hi0 >> (8 * m)) & 0xFFu);
            c[8 + 2 * m] = (float)((lo1 >> (8 * m)) & 0xFFu);
            c[8 + 2 * m + 1] = (float)((hi1 >> (8 * m)) & 0xFFu);
        }
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const float w = wbuf[e * GB + h];
            const float ws = w * sf;
            zacc[h] = fmaf(w, zf, zacc[h]);
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[h][j] = fmaf(ws, c[j], acc[h][j]);
        }
    }
    // reduce over the 8 entry lanes (lane bits 3..5) of each wave
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            zacc[h] += __shfl_xor(zacc[h], o);
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[h][j] += __shfl_xor(acc[h][j], o);
        }
    }
    __syncthreads();  // wbuf reused for the cross-wave reduction
    if (eg == 0) {
#pragma unroll
        for (int h = 0; h < GB; ++h) {
#pragma unroll
            for (int j = 0; j < 16; ++j) wbuf[((wave * GB + h) * 8 + sub) * 17 + j] = acc[h][j];
            wbuf[((wave * GB + h) * 8 + sub) * 17 + 16] = zacc[h];
        }
    }
    __syncthreads();
    for (int o = tid; o < GB * kD; o += kBlock) {
        const int h = o / kD, d = o - h * kD;
        const int sb = d >> 4, j = d & 15;
        float v = 0.0f, z = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            v += wbuf[((w * GB + h) * 8 + sb) * 17 + j];
            z += wbuf[((w * GB + h) * 8 + sb) * 17 + 16];
        }
        p.po[((bh0 + h) * g.NC + chunk) * kD + d] = v + z;
    }
    if (tid < GB) {
        p.pm[(bh0 + tid) * g.NC + chunk] = mh[tid];
        p.pl[(bh0 + tid) * g.NC + chunk] = lh[tid];
    }
}

// ---------------------------------------------------------------------------------------
// Split-K merge: out = sum_c a_c o_c / sum_c a_c l_c, a_c = exp2((m_c - M) log2e/sqrt(D)).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_merge(MergeParams p)
{
    const DecodeGeom &g = p.g;
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const size_t bh = (size_t)b * g.Hq + h;
    const int L = g.seq_lens[b];
    const int nch = L > 0 ? (L + g.CH - 1) >> g.logCH : 0;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, p.pm[bh * g.NC + c]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
        for (int c = 0; c < nch; ++c) {
            const float m = p.pm[bh * g.NC + c];
            if (m == -INFINITY) continue;
            const float a = exp2f((m - M) * p.klog);
            num = fmaf(a, p.po[(bh * g.NC + c) * kD + d], num);
            den = fmaf(a, p.pl[bh * g.NC + c], den);
        }
    }
    p.out[bh * kD + d] = den > 0.0f ? num / den : 0.0f;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_qprep(const QprepParams &p, hipStream_t s)
{
    const float isd = (float)(1.0 / sqrt((double)kD));
    hipLaunchKernelGGL(k_qprep, dim3(p.BH), dim3(128), 0, s, p, isd);
    return hipGetLastError();
}

hipError_t launch_score(const ScoreParams &p, hipStream_t s)
{
    const dim3 grid(p.g.NC, p.g.Hkv * p.g.nsub, p.g.B);
    switch (p.g.GB) {
    case 1: hipLaunchKernelGGL(k_score<1>, grid, dim3(kBlock), 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_score<2>, grid, dim3(kBlock), 0, s, p); break;
    default: hipLaunchKernelGGL(k_score<4>, grid, dim3(kBlock), 0, s, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_bin_scores(const BinScoresParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_bin_scores, dim3(p.g.NC, p.g.Hq, p.g.B), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_hist(const HistParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_hist, dim3(p.nsplit, p.g.Hq, p.g.B), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_threshold(const ThresholdParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_threshold, dim3(p.g.Hq, p.g.B), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_select(const SelectParams &p, hipStream_t s)
{
    const dim3 grid(p.g.NC, p.g.Hq, p.g.B);
    hipLaunchKernelGGL(k_sel_count, grid, dim3(kBlock), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sel_write, grid, dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_attend(const AttendParams &p, bool select, hipStream_t s)
{
    const dim3 grid(p.g.NC, p.g.Hkv * p.g.nsub, p.g.B);
    const dim3 blk(kBlock);
    if (select) {
        switch (p.g.GB) {
        case 1: hipLaunchKernelGGL((k_attend<1, true>), grid, blk, 0, s, p); break;
        case 2: hipLaunchKernelGGL((k_attend<2, true>), grid, blk, 0, s, p); break;
        default: hipLaunchKernelGGL((k_attend<4, true>), grid, blk, 0, s, p); break;
        }
    } else {
        switch (p.g.GB) {
        case 1: hipLaunchKernelGGL((k_attend<1, false>), grid, blk, 0, s, p); break;
        case 2: hipLaunchKernelGGL((k_attend<2, false>), grid, blk, 0, s, p); break;
        default: hipLaunchKernelGGL((k_attend<4, false>), grid, blk, 0, s, p); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_merge, dim3(p.g.Hq, p.g.B), dim3(kD), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvc
