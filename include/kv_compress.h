/*
 * kv_compress.h -- C ABI of the MI355X (gfx950) compressed-KV decode-attention library
 * (libkvcompress.so).
 *
 * The method (from the pages "H1B-KV: Hybrid One-Bit Caches for Memory-Efficient Large
 * Language Model Inference" and "RaBitQCache: Rotated Binary Quantization for KVCache in
 * Long Context LLM Inference"):
 *   - each cached key is stored as the sign bits of a seeded random rotation of the key
 *     (H1B-KV key design: 1-bit sketch by random projection; RaBitQCache abstract:
 *     randomized rotated binary quantization), plus a binary16 norm and a binary16
 *     correction scalar <sign(k')/sqrt(D), k'/|k|>;
 *   - each cached value is stored as per-group 4-bit linear codes with a binary16 scale and
 *     zero point per group (H1B-KV key design);
 *   - at decode the query is rotated and quantized to int4, and the proxy score of every
 *     cached token is formed by binary x INT4 arithmetic (RaBitQCache key design);
 *   - an optional adaptive Top-p keeps the smallest set of tokens whose softmax mass reaches
 *     p (RaBitQCache abstract), and the output is the softmax-weighted sum of the decoded
 *     4-bit values (H1B-KV technical framework: weights from the sketch, output from the
 *     4-bit values).
 *
 * Conventions for every call:
 *   - Pointers are device memory unless marked [host].  The caller allocates and frees all
 *     memory and keeps it alive until the work enqueued on `stream` has completed.  The
 *     library allocates nothing, keeps no pointer after returning, and never synchronizes.
 *   - Each call validates its arguments on the host first.  On a bad argument it returns a
 *     negative code, records a message for kv_last_error(), and enqueues nothing.  A failed
 *     kernel launch returns KV_ERR_HIP with the HIP error string.
 *   - Device-side preconditions are not checked by default: sequence lengths within the pages
 *     the page table maps, page ids < num_pages, finite inputs, and (for append) positions
 *     that stay inside the mapped pages.  With the environment variable KV_DEBUG set to 1 (read
 *     at every call), kv_compress_append and the decode calls first run a checker kernel over
 *     seq_lens, start_pos and the page table entries the call would use (it reads them within
 *     their declared extents only), synchronize `stream`, and return KV_ERR_ARG with the first
 *     offending (sequence, page index, value) in kv_last_error() before enqueuing any other
 *     kernel; such calls are then synchronous and must not be captured into a graph.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the null stream).
 *   - head_dim D must be 128; value_group must be 32 or 64; page_size must be a power of
 *     two >= 16; the GQA group Hq/Hkv must be 1, 2, 4 or 8.
 */
#ifndef KV_COMPRESS_H
#define KV_COMPRESS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KV_OK = 0,
    KV_ERR_ARG = -1,          /* NULL pointer, non-positive size, inconsistent shapes, bad p */
    KV_ERR_UNSUPPORTED = -2,  /* a head_dim, value group, page size or GQA group with no kernel */
    KV_ERR_WORKSPACE = -3,    /* workspace smaller than the *_workspace_bytes() figure */
    KV_ERR_HIP = -4           /* a HIP launch failed; kv_last_error() has the HIP message */
};

enum { KV_ROT_DENSE = 0, KV_ROT_HADAMARD = 1 };
enum { KV_F16 = 0, KV_F32 = 1 };

/* Paged packed cache ([host] struct describing device arrays).
 * Token t of sequence b lives in physical page page_table[b][t / page_size], slot
 * t % page_size; the record of (page p, KV head h, slot s) has index
 * i = (p * num_kv_heads + h) * page_size + s in each of the two arrays:
 *   keys  uint32 [num_pages][Hkv][page_size][S/32 + 1], a 20-byte record per key (12 bytes
 *         for S = 64), with S = sketch_dim (the sign bits per key, D unless set to 64):
 *         words 0..S/32-1: bit r of the rotated key k' = R k is bit r%32 of word r/32, set
 *           when k'_r >= 0, for r < S.  Read as little-endian bytes this is byte r/8, bit
 *           r%8, set = +1: the bitmap order of the H1IB-KV page, section 二.3.
 *         word S/32: binary16 |k| in the low half, binary16 correction
 *           sum_{r<S} |k'_r| / (sqrt(S) |k|) in the high half (1.0 for k = 0).
 *   S < D is a narrow sketch, the non-square random projection onto the first S rows of R
 *   (H1B-KV key design: a 1-bit key sketch by random projection): the query is quantized
 *   over the same S coordinates and the estimator keeps its form with S in place of D in
 *   its sign part (x = sign(k'_{<S})/sqrt(S)); the softmax temperature stays 1/sqrt(D).
 *   vals  uint8 [num_pages][Hkv][page_size][D/2 + 4 D/value_group], a record per value:
 *         bytes 0..D/2-1: 4-bit codes, dim 2m in the low nibble of byte m and dim 2m+1 in
 *           the high nibble;
 *         then one uint32 per group of value_group dims: binary16 scale in the low half,
 *           binary16 zero point in the high half; value = code * scale + zero.
 * A key and a value are each one contiguous record (20 or 12 and 80 or 72 bytes), so that a
 * decode that gathers a few selected tokens touches one or two 128-byte lines per record
 * rather than one per field.
 * keys_f16 (nullable): binary16 [num_pages][Hkv][page_size][D], the keys themselves (not
 *   rotated), rounded to nearest even from binary32 input; 16-byte aligned.  When present,
 *   appends fill it, and a Top-p decode scores the selected tokens exactly with it (the
 *   proxy scores still choose them): RaBitQCache's abstract, proxy scores that estimate the
 *   attention weights to retrieve a token set for sparse attention.  A caller that wants the
 *   proxy scores for a cache that has the array passes a copy of the struct with it NULL.
 * key_center (nullable): binary32 [Hkv][D], 16-byte aligned, one center c_h per KV head (for
 *   instance the mean of the head's keys): per-head key centering before the rotation, an
 *   estimator variant outside the pages.  Appends encode k - c_h (the input widened to
 *   binary32, then one binary32 subtraction per dim) in place of k: the sign bits, the norm
 *   and the correction are those of k - c_h, and keys_f16 still holds k.  The proxy scores
 *   then estimate <q, k - c_h> = <q, k> - <q, c_h>, which differs from <q, k> by one
 *   constant per (sequence, query head); softmax weights do not see such a shift, so the
 *   decode uses the centered scores as they are (Top-p bins included).  Only tail tokens
 *   (kv_decode_attend_tail), scored exactly, are moved into the same frame: <q, k> - <q, c_h>
 *   (unless the cache's exact scores are in use, which are uncentered).  The same centers
 *   must be used for every append and decode of one cache.
 * rot: KV_ROT_DENSE -> binary16 [D][D] row-major orthogonal matrix R (k' = R k);
 *      KV_ROT_HADAMARD -> uint32 [D/32] random signs (bit j set: sigma_j = -1), and
 *      R = H diag(sigma) / sqrt(D) with H the Sylvester-order Hadamard matrix.
 * The same rotation must be used for appends and decodes of one cache. */
typedef struct kv_cache {
    int32_t head_dim;      /* D */
    int32_t num_kv_heads;  /* Hkv */
    int32_t value_group;   /* 32 or 64 dims per scale/zero pair */
    int32_t page_size;     /* tokens per page */
    int32_t num_pages;     /* physical pages in the pool; num_pages * num_kv_heads * page_size
                              must stay below 2^32 (KV_ERR_UNSUPPORTED otherwise) */
    int32_t rot_kind;      /* KV_ROT_DENSE or KV_ROT_HADAMARD */
    const void *rot;       /* device: see above */
    uint32_t *keys;        /* device, 4-byte aligned: see above */
    uint8_t *vals;         /* device, 4-byte aligned: see above */
    uint16_t *keys_f16;    /* device, nullable, 16-byte aligned: see above */
    const float *key_center; /* device, nullable, 16-byte aligned: see above */
    int32_t sketch_dim;    /* sign bits per key: 0 or D (the whole rotation), or 64 */
} kv_cache;

/* Optional intermediate outputs of kv_decode_attend ([host] struct; every member is a
 * nullable device pointer).  Used by tests to compare each stage with the oracle; passing
 * NULL (or NULL members) skips the extra work.  ld = max_seq_len.
 *   q_codes  uint8 [B][Hq][D]       int4 codes u of the rotated query
 *   q_params float [B][Hq][4]       v_l, delta, c0 = v_l/sqrt(D), c1 = delta/sqrt(D)
 *   q_sumu   int32 [B][Hq]          sum of the codes
 *   iscores  int32 [B][Hq][ld]      A = sum_r s_r u_r, s_r = +-1 from the key bits
 *   scores   float [B][Hq][ld]      proxy scores (estimates of <k, q>)
 *   sel_count int32 [B][Hq]         Top-p only: number of selected tokens
 *   sel_idx  int32 [B][Hq][ld]      Top-p only: selected token indices, ascending
 *   sel_bins int32 [B][Hq][2]       Top-p only: top bin e_max and threshold bin distance b*
 *   stage_events [host] array of 2 * KV_NUM_STAGES hipEvent_t (nullable): the call records
 *            stage_events[2s] on `stream` before the kernels of stage s and
 *            stage_events[2s+1] after them, for each stage s it runs (others are left
 *            alone), so a caller can time every stage with hipEventElapsedTime.
 *   bin_dist uint16 [B][Hq][ld]     Top-p only: what the score pass wrote for token t, the
 *            distance chunk_top - e_t of its score bin e_t = floor(s_t * kbin) (see
 *            kv_topp_select) to the top bin of its 512-token chunk, saturated at 8192, and 8192
 *            for positions past seq_lens[b] inside the sequence's last chunk (later chunks are
 *            left undefined).  Copied from the workspace after the score pass, so a decode
 *            without scores/iscores is checked on the very kernels it runs otherwise.
 *   chunk_top int32 [B][Hq][ceil(ld / 512)]  Top-p only: the top bin of each 512-token chunk
 *            (undefined for chunks past seq_lens[b]). */
enum {
    KV_STAGE_QUERY = 0,   /* query rotation, int4 codes, bit-planes */
    KV_STAGE_SCORE = 1,   /* Top-p: proxy scores of all tokens -> bin distances */
    KV_STAGE_HIST = 2,    /* Top-p: per-bin token counts, then the threshold bin */
    KV_STAGE_SELECT = 3,  /* Top-p, only when sel_idx is requested: ordered index lists */
    KV_STAGE_ATTEND = 4,  /* scores of the attended tokens, softmax, 4-bit value sums */
    KV_STAGE_MERGE = 5,   /* merge of the per-chunk partial results */
    KV_NUM_STAGES = 6
};
typedef struct kv_debug {
    uint8_t *q_codes;
    float *q_params;
    int32_t *q_sumu;
    int32_t *iscores;
    float *scores;
    int32_t *sel_count;
    int32_t *sel_idx;
    int32_t *sel_bins;
    hipEvent_t *stage_events;
    uint16_t *bin_dist;
    int32_t *chunk_top;
} kv_debug;

/* kv_compress_append -- encode n_new new tokens per sequence into the cache.
 * Defines: H1B-KV key design (1-bit key sketch by random projection, 4-bit linear values)
 * with RaBitQCache's randomized rotation (abstract).
 *   c          [host] cache descriptor
 *   dtype      KV_F16 or KV_F32: element type of k and v
 *   k, v       [B][n_new][Hkv][D] row-major
 *   start_pos  int32 [B]: token index of the first new token of each sequence
 *   page_table int32 [B][max_pages]
 * Token i of sequence b is written at position start_pos[b] + i.  Appending a sequence in
 * several calls gives the same bytes as one call. */
int kv_compress_append(const kv_cache *c, int32_t dtype, const void *k, const void *v, int32_t B,
                       int32_t n_new, const int32_t *start_pos, const int32_t *page_table,
                       int32_t max_pages, hipStream_t stream);

/* kv_decode_attend -- one decode step of attention over the compressed cache.
 * Defines: H1B-KV technical framework (attention weights from the 1-bit sketch, output
 * from the 4-bit values); RaBitQCache abstract and key design (int4 query, binary x INT4
 * proxy score, adaptive Top-p).
 *   q           float [B][Hq][D]; query head h attends KV head h * Hkv / Hq
 *   seq_lens    int32 [B]: tokens 0..seq_lens[b]-1 of sequence b are attended; must be
 *               <= max_seq_len; a zero length gives a zero output
 *   max_seq_len [host] upper bound of seq_lens (sizes the grid and the workspace)
 *   top_p       [host] >= 1: softmax over all tokens; in (0, 1): adaptive Top-p, then the
 *               softmax renormalised over the selected tokens.  <= 0 or NaN is an error.
 *               Under Top-p with c->keys_f16 set, the softmax over the selected tokens uses
 *               the exact scores <q, k> of their binary16 keys instead of the proxy scores.
 *               B and Hq must be at most 65535 (else KV_ERR_UNSUPPORTED).
 *   out         float [B][Hq][D]
 *   dbg         [host] nullable, see kv_debug
 *   workspace   device scratch of at least kv_decode_workspace_bytes(...) bytes; its
 *               contents on entry do not matter
 * Softmax weights are exp(score / sqrt(D)). */
int kv_decode_attend(const kv_cache *c, const float *q, int32_t B, int32_t Hq,
                     const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                     int32_t max_pages, float top_p, float *out, const kv_debug *dbg,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Uncompressed recent tokens ([host] struct describing device arrays), for lazy updates:
 * RaBitQCache's abstract names asynchronous pipelining and lazy updates that hide the
 * system's overhead.  The newest tokens of each sequence stay in binary16 until a whole
 * page of them is compressed with kv_compress_append (for instance on a second stream,
 * while decodes go on), so a decode step appends nothing to the compressed cache.
 *   k, v      binary16 [B][capacity][Hkv][D], 16-byte aligned: token j of sequence b's
 *             tail at [b][j]; the layout of kv_compress_append's input, so a full page
 *             of the tail is compressed in place (k = tail k + b * capacity * Hkv * D)
 *   len       int32 [B]: tokens in the tail of each sequence, 0 <= len[b] <= capacity
 *   capacity  tokens per sequence in k and v (>= 1) */
typedef struct kv_tail {
    uint16_t *k;
    uint16_t *v;
    int32_t *len;
    int32_t capacity;
    float *mass;           /* nullable float [B][capacity][Hkv]: attention mass accumulated by the
                              decodes of kv_decode_attend_ex with a high-precision tier (the sum
                              over the KV head's query heads of each step's softmax weight);
                              kv_tail_append zeroes it for new tokens, kv_tail_retire moves it */
} kv_tail;

/* High-precision tier ([host] struct describing device arrays): H1IB-KV's high-precision
 * layer, which keeps the most important key-value pairs in binary16 while the rest go to
 * the one-bit layer.  Importance is read here as accumulated attention mass, and a token
 * can enter the tier only while it is still in binary16, i.e. when its page of the tail is
 * compressed (kv_hp_update).  Per (sequence b, KV head h) up to `capacity` entries:
 *   k, v   binary16 [B][Hkv][capacity][D], 16-byte aligned
 *   pos    int32 [B][Hkv][capacity]: the token position of the entry, -1 for an empty one
 *   saved  uint32 [B][Hkv][capacity]: the norm/correction word of the token's compressed
 *          key record, which holds the marker 0x7E007E00 (binary16 NaN norm) while the
 *          token is in the tier; a decode gives a marked record no weight, so the token is
 *          attended once, exactly, from the tier.  Eviction restores the word.
 *   mass   float [B][Hkv][capacity]: accumulated attention mass of the entry
 * All-empty is pos = -1 everywhere (mass and saved are then ignored). */
typedef struct kv_hp {
    uint16_t *k;
    uint16_t *v;
    int32_t *pos;
    uint32_t *saved;
    float *mass;
    int32_t capacity;
} kv_hp;

/* kv_tail_append -- write n_new new tokens per sequence into the tail (lazy update).
 *   dtype  KV_F16 or KV_F32 (rounded to binary16, nearest even)
 *   k, v   [B][n_new][Hkv][D] row-major, Hkv = c->num_kv_heads of the cache they belong to
 * Token i of sequence b goes to tail position len[b] + i, then len[b] += n_new.  Device-side
 * precondition: len[b] + n_new <= capacity (tokens past the capacity are dropped). */
int kv_tail_append(const kv_tail *t, int32_t num_kv_heads, int32_t head_dim, int32_t dtype, const void *k,
                   const void *v, int32_t B, int32_t n_new, hipStream_t stream);

/* kv_tail_retire -- drop the first n tokens of every sequence's tail once they have been
 * compressed into the cache (kv_compress_append on tail positions 0..n-1, which may run on
 * another stream; the caller orders the two).  The remaining tokens move to the front,
 * len[b] -= n, and seq_lens[b] += n when seq_lens (int32 [B], nullable) is given.
 * Device-side precondition: len[b] >= n. */
int kv_tail_retire(const kv_tail *t, int32_t num_kv_heads, int32_t head_dim, int32_t B, int32_t n,
                   int32_t *seq_lens, hipStream_t stream);

/* kv_decode_attend_tail -- kv_decode_attend over a compressed cache plus a binary16 tail.
 * Defines: RaBitQCache abstract (lazy updates); H1B-KV technical framework.
 * Sequence b's context is its seq_lens[b] compressed tokens followed by its tail->len[b]
 * tail tokens.  The compressed tokens are handled exactly as by kv_decode_attend (all of
 * them, or the Top-p set chosen among them; with c->keys_f16, exact scores for that set);
 * every tail token is attended with its exact score <q, k> and its binary16 value.  One
 * softmax spans both.  Arguments and errors as kv_decode_attend, plus a NULL or invalid
 * tail (KV_ERR_ARG); the workspace is kv_decode_workspace_bytes(...) bytes. */
int kv_decode_attend_tail(const kv_cache *c, const kv_tail *tail, const float *q, int32_t B, int32_t Hq,
                          const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                          int32_t max_pages, float top_p, float *out, const kv_debug *dbg,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Optional inputs of a decode step ([host] struct; every member is nullable).
 *   tail      as for kv_decode_attend_tail
 *   q_dither  device float [B][Hq][D]: uniforms U in [0, 1) drawn by the caller, one per
 *             query dim.  The int4 query codes become u_j = clamp(floor(t_j + U_j), 0, 15)
 *             with t_j = (q'_j - v_l) / delta and a binary32 add, in place of rint(t_j):
 *             seeded stochastic rounding, so that E[u_j] = t_j and the query quantization
 *             adds no bias to the proxy score (an estimator variant outside the pages, the
 *             randomized query quantization of RaBitQ).  Values outside [0, 1) are the
 *             caller's error; the codes stay clamped to 0..15. */
/* New tokens that a decode step appends to the cache itself (kv_decode_opts.append): the
 * arguments of kv_compress_append for the decode's B, page_table and max_pages.  The
 * tokens are written exactly as kv_compress_append would write them, before any of them
 * is read, so seq_lens must already count them.  With the randomized Hadamard rotation, or
 * the dense one and at most 8192 new token-heads, the encoding runs inside the decode's
 * first launch, next to the query preparation; otherwise as its own launch first. */
typedef struct kv_append_args {
    int32_t dtype;               /* KV_F16 or KV_F32 */
    const void *k, *v;           /* [B][n_new][Hkv][D] */
    int32_t n_new;               /* >= 0 */
    const int32_t *start_pos;    /* int32 [B] */
} kv_append_args;

typedef struct kv_decode_opts {
    const kv_tail *tail;
    const float *q_dither;
    const kv_hp *hp;       /* nullable: the high-precision tier.  Its entries of KV head h are
                              attended with exact scores and binary16 values in the same softmax
                              as the cache and the tail (scores in the centered frame when the
                              cache has key centers and is scored by proxy); afterwards every
                              tail token and tier entry adds its softmax weight, summed over the
                              KV head's query heads, to its mass (tail->mass must then be set). */
    const kv_append_args *append; /* nullable: new tokens appended first, see kv_append_args */
} kv_decode_opts;

/* kv_decode_attend_ex -- kv_decode_attend with the options of kv_decode_opts (opts NULL or
 * all members NULL: the same as kv_decode_attend).  Arguments, errors and workspace as
 * kv_decode_attend_tail when a tail is given, else as kv_decode_attend. */
int kv_decode_attend_ex(const kv_cache *c, const kv_decode_opts *opts, const float *q, int32_t B, int32_t Hq,
                        const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                        int32_t max_pages, float top_p, float *out, const kv_debug *dbg,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* kv_decode_attend_noalloc -- kv_decode_attend_ex without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a 64 MiB array in the library's device code, one
 * copy per device, held from the library's load until the process ends; its address is taken
 * once per device (hipGetSymbolAddress, with that device current) on the first call that runs
 * on the device.  The call allocates nothing and frees nothing.
 *   Arguments, results and errors as kv_decode_attend_ex; KV_ERR_WORKSPACE when the decode
 *   needs more than 64 MiB of workspace (kv_decode_workspace_bytes(...) > 64 MiB; for example
 *   the 128k-token, 4-sequence, 32-query-head Top-p decode needs about 49 MiB).
 *   Every call on one device shares that device's array, and each call overwrites what it
 *   needs (nothing has to start at zero): calls that may overlap on one device -- on two
 *   streams, or from two threads -- race, and the caller must order them. */
int kv_decode_attend_noalloc(const kv_cache *c, const kv_decode_opts *opts, const float *q, int32_t B, int32_t Hq,
                             const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                             int32_t max_pages, float top_p, float *out, const kv_debug *dbg, hipStream_t stream);

/* kv_hp_update -- the tier's promotion step, when the first n tokens of every tail (positions
 * seq_lens[b] .. seq_lens[b] + n - 1) have been compressed into the cache and before
 * kv_tail_retire(n) drops them.  For each (sequence, KV head), among the tier's entries and
 * those n tokens, the `capacity` with the largest mass stay or enter (ties: the lower
 * position first; empty entries last).  An entering token's binary16 key and value are
 * copied from the tail, its mass carried over, and its compressed key record marked (the
 * old word kept in saved); a leaving entry's record word is restored and the entry emptied.
 *   c          the cache the tokens were compressed into (page_table as for the append)
 *   seq_lens   int32 [B]: compressed tokens before the n, as kv_tail_retire will advance them
 * Requires t->mass, n <= t->capacity and capacity + n <= 1024. */
int kv_hp_update(const kv_cache *c, const kv_hp *hp, const kv_tail *t, int32_t B, int32_t n,
                 const int32_t *seq_lens, const int32_t *page_table, int32_t max_pages, hipStream_t stream);

/* Workspace size for kv_decode_attend, kv_decode_attend_tail and kv_decode_attend_ex with these
 * arguments (0 on invalid arguments).  kv_workspace_bytes is the same function under the name
 * the decode's statement of the problem uses; kv_topp_select has a sizer of its own
 * (kv_topp_workspace_bytes), since it takes scores rather than a cache. */
size_t kv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len,
                                 int32_t head_dim, float top_p);
size_t kv_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len, int32_t head_dim,
                          float top_p);

/* kv_topp_select -- adaptive Top-p over caller-supplied proxy scores.
 * Defines: RaBitQCache abstract (adaptive Top-p retrieval whose token budget follows the
 * actual attention sparsity), read as the textbook nucleus evaluated on integer weights:
 *   bin e_i = floor(s_i * kbin), kbin = fp32(256 log2(e) / sqrt(head_dim)), clamped to
 *   [-2^29, 2^29]; d_i = max_j e_j - e_i; weight W(d) = T[d mod 256] >> (d / 256) for
 *   d < 8192 and 0 beyond, T[j] = round(2^(32 - j/256)); Z = sum_i W(d_i);
 *   T_p = ceil(Z * rint(p * 2^24) / 2^24); b* = min { b : sum_{d_i <= b} W(d_i) >= T_p };
 *   selected set S = { i : d_i <= b* }.  When e_max itself is the bottom bin -2^29 (every
 *   score NaN or below -2^29 / kbin: no token has weight), S is empty.
 *   scores    float [B][Hq][ld]; tokens 0..seq_lens[b]-1 are used (seq_lens <= ld)
 *   top_p     [host] in (0, 1)
 *   sel_idx   int32 [B][Hq][ld]: S in ascending order; entries past the count are untouched
 *   sel_count int32 [B][Hq]
 *   workspace at least kv_topp_workspace_bytes(B, Hq, ld) bytes */
int kv_topp_select(const float *scores, int32_t ld, const int32_t *seq_lens, int32_t B,
                   int32_t Hq, int32_t head_dim, float top_p, int32_t *sel_idx,
                   int32_t *sel_count, void *workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Workspace size for kv_topp_select (0 on invalid arguments). */
size_t kv_topp_workspace_bytes(int32_t B, int32_t Hq, int32_t ld);

/* Message describing the last error of this thread (static storage; "" if none). */
const char *kv_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int kv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KV_COMPRESS_H */
