/*
 * kvc_oracle.c -- reference ("oracle") implementation of decode attention over a
 * 1-bit-key / 4-bit-value compressed KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This is plain, slow, single-threaded C99 that writes each step
 * of the method out directly, so that a reader can check it against the pages by eye.  Only
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the GPU library, and the GPU library never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [H1B]   "H1B-KV: Hybrid One-Bit Caches for Memory-Efficient Large Language Model
 *           Inference" -- abstract; "technical framework" (attention weights come from the
 *           1-bit key sketch, the output from the 4-bit values); "key design" (1-bit key
 *           sketch by random projection, 4-bit *linear* quantization of values).
 *   [RBQC]  "RaBitQCache: Rotated Binary Quantization for KVCache in Long Context LLM
 *           Inference" -- abstract and "key design": randomized rotation + binary
 *           quantization of keys, binary x INT4 arithmetic for the proxy score, the proxy
 *           score is an unbiased estimator, adaptive Top-p retrieval.
 *   [H1IB]  "混合单比特缓存技术：H1IB-KV助力大模型推理内存优化" -- section 二.1 (sign function
 *           gives +-1) and section 二.3 (bitmap: element idx lives in byte idx/8, bit idx%8,
 *           a set bit means +1).
 *   [RaBitQ, outside the pages] Gao & Long, "RaBitQ", SIGMOD 2024: the form of the
 *           unbiased estimator <k,q> ~ |k| <x, q'> / <x, k'/|k|>, x = sign(k')/sqrt(D).
 *
 * Precision.  Where a step has a plain mathematical definition the oracle evaluates it in
 * binary64 (key rotation, norms, the attention softmax and weighted sum).  Where a floating
 * point result decides an integer (the int4 query codes, the value codes, the Top-p bin of
 * a score) the pages fix no precision, so the oracle takes that decision in binary32 with
 * the operation order stated at each function -- the precision the GPU kernels use.
 *
 * Build: gcc -O2 -std=gnu11 -ffp-contract=off -fPIC -shared (no -ffast-math; x86-64 SSE2
 * arithmetic has no excess precision).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ROT_DENSE 0
#define ORC_ROT_HADAMARD 1

/* ------------------------------------------------------------------------------------- */
/* IEEE binary16 conversions (round to nearest, ties to even).                            */
/* ------------------------------------------------------------------------------------- */

/* binary64 -> binary16, correctly rounded.  A binary32 input is passed as its exact
 * binary64 value, so this also gives the correctly rounded binary32 -> binary16. */
uint16_t orc_f16_from_f64(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs(x);
    /* The largest finite half is 65504; anything at or above the midpoint to 65536 rounds
     * to infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int E;
    frexp(a, &E);          /* a = m * 2^E, m in [0.5, 1): a lies in [2^(E-1), 2^E) */
    int e = E - 1;
    if (e < -14) e = -14;  /* subnormals share the quantum 2^-24 of the smallest binade */
    /* number of quanta 2^(e-10), rounded to nearest even (default rounding mode) */
    double q = nearbyint(ldexp(a, 10 - e));
    /* q in [0, 2048]; q >= 1024 is a normal number of exponent e (q == 2048 carries into
     * exponent e+1 with a zero fraction); for e == -14, q < 1024 is a subnormal. */
    int bits = ((e + 15) << 10) + (int)q - 1024;
    return (uint16_t)(sign | (uint16_t)bits);
}

double orc_f64_from_f16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 1024), e - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------------------- */
/* Random rotation (keys: binary64).                                                      */
/* ------------------------------------------------------------------------------------- */

/* Sylvester (natural-order) Hadamard entry H[r][j] = (-1)^popcount(r & j). */
static int hadamard_entry(int r, int j)
{
    return (__builtin_popcount((unsigned)(r & j)) & 1) ? -1 : 1;
}

/* Random sign j of the randomized Hadamard rotation: bit j of the sign words; a set bit
 * means sigma_j = -1. */
static int sigma_is_negative(const uint32_t *signs, int j)
{
    return (int)((signs[j >> 5] >> (j & 31)) & 1u);
}

/* y = R x in binary64.
 *   dense:    R is a D x D orthogonal matrix stored in binary16 (passed here as the float
 *             values of its entries, row-major): y_r = sum_j R[r][j] x_j.
 *   hadamard: R = H diag(sigma) / sqrt(D):          y_r = sum_j H[r][j] sigma_j x_j / sqrt(D).
 * A random rotation followed by a sign is the 1-bit sketch ([RBQC] abstract: "randomized
 * rotated binary quantization"; [H1B] key design: "random projection").  The plain O(D^2)
 * sum is used on purpose: for binary16 inputs every partial sum is exact in binary64, so
 * the sign of y_r is that of the exact product. */
static void rotate_f64(int D, int rot_kind, const float *R, const uint32_t *signs,
                       const float *x, double *y)
{
    for (int r = 0; r < D; ++r) {
        double acc = 0.0;
        for (int j = 0; j < D; ++j) {
            if (rot_kind == ORC_ROT_DENSE) {
                acc += (double)R[(size_t)r * D + j] * (double)x[j];
            } else {
                double xj = sigma_is_negative(signs, j) ? -(double)x[j] : (double)x[j];
                acc += hadamard_entry(r, j) * xj;
            }
        }
        y[r] = (rot_kind == ORC_ROT_DENSE) ? acc : acc / sqrt((double)D);
    }
}

/* Exported for tests: y = R x in binary64. */
void orc_rotate_f64(int D, int rot_kind, const float *R, const uint32_t *signs,
                    const float *x, int64_t n, double *y)
{
    for (int64_t i = 0; i < n; ++i)
        rotate_f64(D, rot_kind, R, signs, x + i * D, y + i * D);
}

/* ------------------------------------------------------------------------------------- */
/* Key encode: sign bits of the rotated key + binary16 norm and correction.               */
/* ------------------------------------------------------------------------------------- */

/* For each of n keys k (D floats), with a sketch of the first sk rotated coordinates
 * (sk = D: the whole rotation; sk < D, a multiple of 32: a non-square random projection,
 * the rows 0..sk-1 of R, read from "H1B-KV" key design as a 1-bit sketch by random
 * projection):
 *   k' = R k                                   (binary64, rotate_f64)
 *   bit_r = 1 if k'_r >= 0 else 0, r < sk      ([H1IB] 二.1: sign gives +-1; a zero counts
 *                                               as +1)
 *   bit r is stored in 32-bit word r/32 at bit position r%32; viewed as little-endian
 *   bytes this is byte r/8, bit r%8, exactly the bitmap order of [H1IB] 二.3.
 *   norm = fp16(|k|_2)                         (the whole key)
 *   corr = fp16( sum_{r<sk} |k'_r| / (sqrt(sk) |k|) ) = fp16(<x, k'/|k|>),
 *          x = sign(k'_{<sk})/sqrt(sk) ([RaBitQ, outside the pages]: the estimator's
 *          normaliser); corr = 1 when k = 0.
 * Output: bits[n][sk/32], nc[n][2] = (norm, corr) as binary16 bit patterns. */
void orc_key_encode(int D, int sk, int rot_kind, const float *R, const uint32_t *signs,
                    const float *k, int64_t n, uint32_t *bits, uint16_t *nc)
{
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    int W = sk / 32;
    for (int64_t i = 0; i < n; ++i) {
        const float *ki = k + i * D;
        rotate_f64(D, rot_kind, R, signs, ki, y);
        uint32_t *bw = bits + i * W;
        for (int w = 0; w < W; ++w) bw[w] = 0u;
        for (int r = 0; r < sk; ++r)
            if (!(y[r] < 0.0)) bw[r >> 5] |= 1u << (r & 31);
        double ss = 0.0, sabs = 0.0;
        for (int j = 0; j < D; ++j) ss += (double)ki[j] * (double)ki[j];
        for (int r = 0; r < sk; ++r) sabs += fabs(y[r]);
        double nrm = sqrt(ss);
        nc[2 * i + 0] = orc_f16_from_f64(nrm);
        nc[2 * i + 1] = orc_f16_from_f64(nrm == 0.0 ? 1.0 : sabs / (sqrt((double)sk) * nrm));
    }
    free(y);
}

/* ------------------------------------------------------------------------------------- */
/* Value encode: per-group asymmetric int4 ([H1B] key design: 4-bit linear quantization). */
/* ------------------------------------------------------------------------------------- */

/* For each of n value vectors v (D floats) and each group g of Gv consecutive dims:
 *   mn = min, mx = max over the group                             (exact)
 *   scale = fp16( (mx - mn) / 15 )   -- binary32 subtract and divide, then to binary16
 *   zero  = fp16( mn )
 *   c_j   = 0                                  if scale == 0
 *         = clamp( rint((v_j - zero) / scale), 0, 15 )  otherwise (binary32 subtract and
 *           divide with the binary16 scale/zero widened to binary32; rint ties to even)
 * The decoded value is c_j * scale + zero.
 * Output: codes[n][D/2] (byte m holds c_{2m} in its low nibble and c_{2m+1} in its high
 * nibble), sz[n][D/Gv][2] = (scale, zero) as binary16 bit patterns. */
void orc_value_encode(int D, int Gv, const float *v, int64_t n, uint8_t *codes, uint16_t *sz)
{
    int ng = D / Gv;
    for (int64_t i = 0; i < n; ++i) {
        const float *vi = v + i * D;
        uint8_t *ci = codes + i * (D / 2);
        for (int m = 0; m < D / 2; ++m) ci[m] = 0;
        for (int g = 0; g < ng; ++g) {
            float mn = vi[g * Gv], mx = vi[g * Gv];
            for (int j = 1; j < Gv; ++j) {
                float x = vi[g * Gv + j];
                if (x < mn) mn = x;
                if (x > mx) mx = x;
            }
            float range = mx - mn;
            float step = range / 15.0f;
            uint16_t s16 = orc_f16_from_f64((double)step);
            uint16_t z16 = orc_f16_from_f64((double)mn);
            float sf = (float)orc_f64_from_f16(s16);
            float zf = (float)orc_f64_from_f16(z16);
            sz[(i * ng + g) * 2 + 0] = s16;
            sz[(i * ng + g) * 2 + 1] = z16;
            for (int j = 0; j < Gv; ++j) {
                int c = 0;
                if (sf != 0.0f) {
                    float t = rintf((vi[g * Gv + j] - zf) / sf);
                    if (t < 0.0f) t = 0.0f;
                    if (t > 15.0f) t = 15.0f;
                    c = (int)t;
                }
                int d = g * Gv + j;
                ci[d >> 1] |= (uint8_t)(c << ((d & 1) * 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------------------- */
/* Query encode: rotate (binary32) and quantize to int4 ([RBQC] binary x INT4).           */
/* ------------------------------------------------------------------------------------- */

/* 1/sqrt(D) rounded to binary32. */
static float inv_sqrt_d(int D) { return (float)(1.0 / sqrt((double)D)); }

/* For each of nq queries q (D floats), in binary32 with this exact operation order (sk:
 * the sketch width of the keys, as for orc_key_encode; only the first sk rotated
 * coordinates are quantized, the codes of the others are 0):
 *   dense:    q'_r = fmaf chain over j ascending: a = R[r][0]*q_0; a = fmaf(R[r][j], q_j, a)
 *   hadamard: x_j = sigma_j q_j; for h = 1, 2, 4, ..., D/2 and every i with (i & h) == 0:
 *             (x_i, x_{i+h}) <- (x_i + x_{i+h}, x_i - x_{i+h})   (the textbook in-place fast
 *             Walsh-Hadamard transform, Sylvester order); q'_j = x_j * fp32(1/sqrt(D))
 *   v_l = min_{j<sk} q'_j, v_r = max_{j<sk} q'_j, delta = (v_r - v_l) / 15
 *   u_j = 0 if delta == 0 or j >= sk, else clamp(rint((q'_j - v_l) / delta), 0, 15)
 *         (ties to even)
 *         or, with dither (uniforms U in [0, 1), one per query dim, nullable):
 *         clamp(floor((q'_j - v_l) / delta + U_j), 0, 15)  (stochastic rounding: the
 *         expected code is (q'_j - v_l) / delta; RaBitQ's randomized query quantization,
 *         outside the pages; binary32 divide, then binary32 add)
 *   c0 = v_l * fp32(1/sqrt(sk)),  c1 = delta * fp32(1/sqrt(sk)),  sumu = sum_j u_j
 * The dequantized query is q'_j ~ v_l + delta u_j, and x = sign(k'_{<sk})/sqrt(sk) gives
 * <x, q> ~ c1 * A + c0 * P with A = sum_{j<sk} s_j u_j, P = sum_{j<sk} s_j, s_j = +-1.
 * Output: u[nq][D] (one code per byte), par[nq][4] = (v_l, delta, c0, c1), sumu[nq],
 * qrot[nq][D] (optional, the rotated query before quantization). */
void orc_query_encode(int D, int sk, int rot_kind, const float *R, const uint32_t *signs,
                      const float *q, int64_t nq, const float *dither, uint8_t *u, float *par,
                      int32_t *sumu, float *qrot)
{
    float *x = (float *)malloc(sizeof(float) * (size_t)D);
    float isd = inv_sqrt_d(D);
    float isk = inv_sqrt_d(sk);
    for (int64_t i = 0; i < nq; ++i) {
        const float *qi = q + i * D;
        if (rot_kind == ORC_ROT_DENSE) {
            for (int r = 0; r < D; ++r) {
                const float *Rr = R + (size_t)r * D;
                float a = Rr[0] * qi[0];
                for (int j = 1; j < D; ++j) a = fmaf(Rr[j], qi[j], a);
                x[r] = a;
            }
        } else {
            for (int j = 0; j < D; ++j) x[j] = sigma_is_negative(signs, j) ? -qi[j] : qi[j];
            for (int h = 1; h < D; h <<= 1)
                for (int a = 0; a < D; ++a)
                    if ((a & h) == 0) {
                        float p0 = x[a], p1 = x[a + h];
                        x[a] = p0 + p1;
                        x[a + h] = p0 - p1;
                    }
            for (int j = 0; j < D; ++j) x[j] = x[j] * isd;
        }
        float vl = x[0], vr = x[0];
        for (int j = 1; j < sk; ++j) {
            if (x[j] < vl) vl = x[j];
            if (x[j] > vr) vr = x[j];
        }
        float delta = (vr - vl) / 15.0f;
        int32_t su = 0;
        for (int j = 0; j < D; ++j) {
            int c = 0;
            if (delta != 0.0f && j < sk) {
                float tq = (x[j] - vl) / delta;
                float t = dither ? floorf(tq + dither[i * D + j]) : rintf(tq);
                if (t < 0.0f) t = 0.0f;
                if (t > 15.0f) t = 15.0f;
                c = (int)t;
            }
            u[i * D + j] = (uint8_t)c;
            su += c;
            if (qrot) qrot[i * D + j] = x[j];
        }
        par[i * 4 + 0] = vl;
        par[i * 4 + 1] = delta;
        par[i * 4 + 2] = vl * isk;
        par[i * 4 + 3] = delta * isk;
        sumu[i] = su;
    }
    free(x);
}

/* ------------------------------------------------------------------------------------- */
/* Proxy score ([RBQC]: binary x INT4 arithmetic; unbiased proxy score).                  */
/* ------------------------------------------------------------------------------------- */

/* For each of L encoded keys (sketches of sk bits) against one encoded query (u[D], c0, c1):
 *   s_j = +1 if bit j is set else -1, j < sk    ([H1IB] 二.3 bit order)
 *   A = sum_{j<sk} s_j u_j,   P = sum_{j<sk} s_j  (integers, written as explicit +-1 dots)
 *   r = float(norm) / float(corr)                 (binary32 divide)
 *   score = fmaf(c1, float(A), c0 * float(P)) * r (binary32; c0*P rounded first)
 * score estimates <k, q>: |k| <x, q'> / <x, k'/|k|>, with <x, q'> ~ c1 A + c0 P. */
void orc_scores(int sk, const uint32_t *bits, const uint16_t *nc, int64_t L,
                const uint8_t *u, float c0, float c1, int32_t *A, int32_t *P, float *score)
{
    int W = sk / 32;
    for (int64_t t = 0; t < L; ++t) {
        const uint32_t *bw = bits + t * W;
        int32_t a = 0, p = 0;
        for (int j = 0; j < sk; ++j) {
            int s = ((bw[j >> 5] >> (j & 31)) & 1u) ? 1 : -1;
            a += s * (int32_t)u[j];
            p += s;
        }
        float nrm = (float)orc_f64_from_f16(nc[2 * t + 0]);
        float cor = (float)orc_f64_from_f16(nc[2 * t + 1]);
        float r = nrm / cor;
        float cp = c0 * (float)p;
        float sc = fmaf(c1, (float)a, cp) * r;
        if (A) A[t] = a;
        if (P) P[t] = p;
        if (score) score[t] = sc;
    }
}

/* ------------------------------------------------------------------------------------- */
/* Adaptive Top-p ([RBQC] abstract: the token budget follows the attention sparsity).     */
/* ------------------------------------------------------------------------------------- */

#define ORC_NBINS 8192
#define ORC_BIN_CLAMP 536870912 /* 2^29 */

/* Bins per unit score: a score s has softmax weight exp(s / sqrt(D)) = 2^(s * kbin / 256),
 * so one bin is a factor 2^(1/256) in weight.  kbin = fp32(256 log2(e) / sqrt(D)). */
float orc_kbin(int D) { return (float)(256.0 * 1.4426950408889634074 / sqrt((double)D)); }

/* Bin of a score: floor(s * kbin) in binary32, clamped to [-2^29, 2^29] (a NaN goes to the
 * bottom). */
int32_t orc_bin(float s, float kbin)
{
    float x = s * kbin;
    if (!(x >= -(float)ORC_BIN_CLAMP)) return -ORC_BIN_CLAMP;
    if (x >= (float)ORC_BIN_CLAMP) return ORC_BIN_CLAMP;
    return (int32_t)floorf(x);
}

/* Bins of L scores: e[i] = orc_bin(s[i], kbin(D)). */
void orc_bins(int D, const float *s, int64_t L, int32_t *e)
{
    float kb = orc_kbin(D);
    for (int64_t i = 0; i < L; ++i) e[i] = orc_bin(s[i], kb);
}

/* Weight table T[j] = round(2^(32 - j/256)), j = 0..255. */
void orc_weight_table(uint64_t *T)
{
    for (int j = 0; j < 256; ++j) T[j] = (uint64_t)llround(ldexp(exp2(-(double)j / 256.0), 32));
}

/* Integer weight of a token d bins below the top bin: T[d mod 256] >> (d / 256) for
 * d < 8192 (a factor 2^(-d/256) of the top weight 2^32, truncated), 0 beyond. */
static uint64_t bin_weight(const uint64_t *T, int64_t d)
{
    if (d >= ORC_NBINS) return 0;
    return T[d & 255] >> (d >> 8);
}

/* Top-p selection over one head's L scores:
 *   e_i = bin(s_i), e_max = max e_i, d_i = e_max - e_i
 *   Z   = sum_i W(d_i)                              (exact, 64-bit)
 *   T_p = ceil(Z * p_fx / 2^24), p_fx = rint(p * 2^24)   (exact, 128-bit product)
 *   b*  = the smallest b with sum_{i : d_i <= b} W(d_i) >= T_p
 *   S   = { i : d_i <= b* }, returned as ascending indices.
 * S is the smallest prefix of bins, heaviest first, whose weight reaches the fraction p of
 * the total: the textbook nucleus, at a resolution of 2^(1/256) in weight.  Whole bins are
 * kept, so equal scores are kept or dropped together.  When e_max is the bottom bin itself
 * (every score NaN, or below -2^29 / kbin), no token has weight and S is empty (b* = -1):
 * NaN scores mark records that the cache holds elsewhere.  Returns |S|; sel_idx may be
 * NULL. */
int64_t orc_topp(int D, const float *s, int64_t L, float p, int32_t *sel_idx,
                 int32_t *emax_out, int32_t *bstar_out, uint64_t *Z_out, uint64_t *Tp_out)
{
    if (L <= 0) return 0;
    uint64_t T[256];
    orc_weight_table(T);
    float kb = orc_kbin(D);
    int32_t emax = orc_bin(s[0], kb);
    for (int64_t i = 1; i < L; ++i) {
        int32_t e = orc_bin(s[i], kb);
        if (e > emax) emax = e;
    }
    if (emax == -ORC_BIN_CLAMP) {
        if (emax_out) *emax_out = emax;
        if (bstar_out) *bstar_out = -1;
        if (Z_out) *Z_out = 0;
        if (Tp_out) *Tp_out = 0;
        return 0;
    }
    /* count of tokens per bin distance d < 8192 */
    uint64_t *cnt = (uint64_t *)calloc(ORC_NBINS, sizeof(uint64_t));
    uint64_t Z = 0;
    for (int64_t i = 0; i < L; ++i) {
        int64_t d = (int64_t)emax - (int64_t)orc_bin(s[i], kb);
        Z += bin_weight(T, d);
        if (d < ORC_NBINS) cnt[d] += 1;
    }
    uint32_t pfx = (uint32_t)rint((double)p * 16777216.0);
    unsigned __int128 prod = (unsigned __int128)Z * pfx;
    uint64_t Tp = (uint64_t)((prod + ((unsigned __int128)1 << 24) - 1) >> 24);
    int64_t bstar = ORC_NBINS - 1;
    uint64_t F = 0;
    for (int64_t b = 0; b < ORC_NBINS; ++b) {
        F += cnt[b] * bin_weight(T, b);
        if (F >= Tp) { bstar = b; break; }
    }
    free(cnt);
    int64_t n = 0;
    for (int64_t i = 0; i < L; ++i) {
        int64_t d = (int64_t)emax - (int64_t)orc_bin(s[i], kb);
        if (d <= bstar) {
            if (sel_idx) sel_idx[n] = (int32_t)i;
            ++n;
        }
    }
    if (emax_out) *emax_out = emax;
    if (bstar_out) *bstar_out = (int32_t)bstar;
    if (Z_out) *Z_out = Z;
    if (Tp_out) *Tp_out = Tp;
    return n;
}

/* ------------------------------------------------------------------------------------- */
/* Attention over the 4-bit values ([H1B] technical framework: weights from the sketch,  */
/* output from the 4-bit values).                                                         */
/* ------------------------------------------------------------------------------------- */

/* out = sum_{i in S} w_i v^_i / sum_{i in S} w_i, in binary64, where
 *   w_i  = exp((s_i - m) / sqrt(D)),  m = max_{i in S} s_i   (scaled dot-product softmax
 *          over the proxy scores, renormalised over S)
 *   v^_ij = c_ij * scale_ig + zero_ig                       (the decoded 4-bit value)
 * S is all L tokens when idx == NULL, else idx[0..n-1].  An empty S gives zeros. */
void orc_attend(int D, int Gv, const float *s, const uint8_t *codes, const uint16_t *sz,
                int64_t L, const int32_t *idx, int64_t n, double *out)
{
    int ng = D / Gv;
    int64_t cnt = idx ? n : L;
    for (int j = 0; j < D; ++j) out[j] = 0.0;
    if (cnt <= 0) return;
    double m = -INFINITY;
    for (int64_t a = 0; a < cnt; ++a) {
        int64_t i = idx ? idx[a] : a;
        if ((double)s[i] > m) m = (double)s[i];
    }
    double rs = 1.0 / sqrt((double)D), l = 0.0;
    for (int64_t a = 0; a < cnt; ++a) {
        int64_t i = idx ? idx[a] : a;
        double w = exp(((double)s[i] - m) * rs);
        l += w;
        for (int j = 0; j < D; ++j) {
            int c = (codes[i * (D / 2) + (j >> 1)] >> ((j & 1) * 4)) & 15;
            int g = j / Gv;
            double sc = orc_f64_from_f16(sz[(i * ng + g) * 2 + 0]);
            double zr = orc_f64_from_f16(sz[(i * ng + g) * 2 + 1]);
            out[j] += w * ((double)c * sc + zr);
        }
    }
    for (int j = 0; j < D; ++j) out[j] /= l;
}
