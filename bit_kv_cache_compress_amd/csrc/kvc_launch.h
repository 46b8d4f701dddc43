// Kernel parameter blocks and launchers of libkvcompress (host <-> kernels interface).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// Stage timing (kv_debug.stage_events): while set, the next kernel this thread launches
// records `start` when it begins, and every kernel it launches records `stop` when it ends
// (hipExtLaunchKernel), so the pair brackets a stage's kernels as a kernel trace does, without
// the dispatch latency of event packets between them.
struct StageTiming {
    hipEvent_t start, stop;
};
extern thread_local StageTiming g_stage_timing;

#define KVC_LAUNCH(kern, grid, block, s, ...)                                                               \
    do {                                                                                                  \
        if (::kvc::g_stage_timing.stop) {                                                                 \
            hipExtLaunchKernelGGL(kern, grid, block, 0, s, ::kvc::g_stage_timing.start,                   \
                                  ::kvc::g_stage_timing.stop, 0, __VA_ARGS__);                            \
            ::kvc::g_stage_timing.start = nullptr;                                                        \
        } else {                                                                                          \
            hipLaunchKernelGGL(kern, grid, block, 0, s, __VA_ARGS__);                                     \
        }                                                                                                 \
    } while (0)

// Tokens per Top-p score chunk (one wave of the score kernel, 8 tokens per lane).
constexpr int kTopPChunk = 512;
// Tokens per Top-p attention chunk (one wave of the attention kernel).
constexpr int kTopPAttendChunk = 1024;
// Most tokens per full-softmax attention chunk (one wave of the attention kernel).
constexpr int kMaxFullChunk = 2048;
// Most chunks per sequence (the merge keeps one weight per chunk in LDS).
constexpr int kMaxChunks = 16384;

// Device view of the paged cache: one key record and one value record per slot.
struct CacheView {
    int Hkv;
    int P;       // page size (power of two)
    int logP;
    int Gv;      // value group (32 or 64)
    int lngrp;   // log2(128 / Gv)
    uint32_t *keys;  // [pages][Hkv][P][5]: 4 sign words, norm/corr word
    uint8_t *vals;   // [pages][Hkv][P][64 + 4 * 128/Gv]: codes, scale/zero words
    uint16_t *kf16;  // nullable [pages][Hkv][P][128]: binary16 keys (unrotated)
    const float *kc; // nullable [Hkv][128]: key centers subtracted before the rotation
    int kw;          // sign words per key record: 4 (the whole rotation) or 2 (a 64-bit sketch)
    int sk;          // sign bits per key: 32 kw
};

// Key record of a slot (kw sign words, then the norm/corr word: 20 or 12 bytes).
__device__ __forceinline__ uint32_t *key_rec(const CacheView &c, size_t slot) { return c.keys + slot * (c.kw + 1); }
// Value record of a slot (64 bytes of codes, then 128/Gv scale/zero words).
__device__ __forceinline__ uint8_t *val_rec(const CacheView &c, size_t slot)
{
    return c.vals + (slot << 6) + (slot << (2 + c.lngrp));
}

struct AppendParams {
    CacheView c;
    int rot_kind;          // 0 dense, 1 hadamard
    const void *rot;       // dense: binary16 [128][128]; hadamard: uint32 [4]
    int dtype;             // 0 f16, 1 f32
    const void *k, *v;     // [B][n_new][Hkv][128]
    int B, n_new;
    const int32_t *start_pos;
    const int32_t *page_table;
    int max_pages;
};

// Attention over the binary16 tail of recent tokens: per query head, the running max m,
// weight sum l and weighted value sum o of its tail tokens.
struct TailParams {
    int B, Hq, G, Hkv;
    float klog;
    const float *q;        // [B*Hq][128]
    const uint16_t *k, *v; // [B][cap][Hkv][128] binary16
    const int32_t *len;    // [B]
    int cap;
    float *tm, *tl, *to;   // [B*Hq], [B*Hq], [B*Hq][128]
    const float *center;   // nullable [Hkv][128]: scores are <q, k> - <q, center> (centered frame)
    const uint16_t *hk, *hv;  // nullable: high-precision tier [B][Hkv][hcap][128] binary16
    const int32_t *hpos;   // [B][Hkv][hcap], -1 = empty
    int hcap;
};

// Accumulation of attention mass into the tail and the high-precision tier, done by the
// merge once the softmax normalizer of each query head is known.
struct MassParams {
    const float *q;        // [B*Hq][128]
    const float *center;   // nullable, as TailParams
    const uint16_t *tk;    // tail keys [B][tcap][Hkv][128]
    const int32_t *tlen;   // [B]
    int tcap;
    float *tmass;          // [B][tcap][Hkv]
    const uint16_t *hk;    // tier keys [B][Hkv][hcap][128]
    const int32_t *hpos;   // [B][Hkv][hcap]
    float *hmass;          // [B][Hkv][hcap]
    int hcap;
};

// Query preparation: rotate, quantize, bit-planes.
struct QprepParams {
    int rot_kind;
    const void *rot;
    const float *q;        // [B*Hq][128]
    int BH;
    uint32_t *qnib;        // [B*Hq][16] int4 codes in dot8 order
    uint8_t *qa;           // [B*Hq][128] codes as the fp8 A operand of the matrix-core score
    float4 *qpar;          // [B*Hq]
    uint8_t *dbg_codes;    // nullable [B*Hq][128]
    float *dbg_params;     // nullable [B*Hq][4]
    int32_t *dbg_sumu;     // nullable [B*Hq]
    int sk;                // sketch width of the keys: dims quantized (the rest code 0)
    float isk;             // fp32(1/sqrt(sk)), the scale of c0, c1
    const float *dither;   // nullable [B*Hq][128]: uniforms of the stochastic rounding
    int has_tail;          // blocks BH .. 2 BH - 1 attend over the binary16 tail
    TailParams tail;
    int32_t *order_ctr;    // nullable [2]: cleared for the threshold pass's dispatch slots
    long app_blocks;       // 0, or the blocks after those that encode new tokens (fused append)
    long app_N;            // token-heads to encode
    AppendParams app;
};

// Chunked decode geometry shared by the decode kernels.
struct DecodeGeom {
    int B, Hq, Hkv;
    int G;        // Hq / Hkv
    int GB;       // query heads per block (<= 4)
    int nsub;     // G / GB
    int CH;       // tokens per chunk (power of two, multiple of 256)
    int logCH;
    int NC;       // chunks per sequence (max)
    int Lpad;     // NC * CH
    int KA;       // score chunks per attention block (Top-p), 1 for full softmax
    int NCA;      // attention chunks per sequence (max) = ceil(NC / KA)
    int ld;       // max_seq_len (row stride of debug/score/index arrays)
    const int32_t *seq_lens;
    const int32_t *page_table;
    int max_pages;
};

struct ScoreParams {
    DecodeGeom g;
    CacheView c;
    const uint32_t *qnib;
    const uint8_t *qa;
    const float4 *qpar;
    float kbin;
    uint16_t *dl;          // nullable [B*Hq][Lpad]: bin distance to the chunk's top bin
    int32_t *lmax;         // nullable [B*Hq][NC]: chunk top bin
    float *dbg_scores;     // nullable [B*Hq][ld]
    int32_t *dbg_iscores;  // nullable [B*Hq][ld]
};

// Bins from caller-supplied scores (kv_topp_select).
struct BinScoresParams {
    DecodeGeom g;          // Hq used as rows; GB = 1
    const float *scores;   // [B*Hq][ld]
    float kbin;
    uint16_t *dl;
    int32_t *lmax;
};

// Histogram of bin distances per split, then the Top-p threshold of each (b, h).
struct HistParams {
    DecodeGeom g;
    int nsplit, cps;       // splits per (b,h), chunks per split
    int fused;             // one block per head counts and thresholds (k_hist_thresh)
    uint32_t pfx;          // rint(p * 2^24)
    const uint16_t *dl;
    const int32_t *lmax;
    uint16_t *hist;        // [B*Hq][nsplit][8192] per-split counts (a split has < 65536 tokens);
                           // splits past a sequence's end are neither written nor read
    int32_t *sel;          // [B*Hq][4] = (e_max, b*, count, 0)
    int32_t *order;        // nullable [B*Hq]: the heads in the attention pass's dispatch order
    int32_t *order_ctr;    // [2] slots taken from the front and from the back of `order`
    int32_t *dbg_count;    // nullable [B*Hq]
    int32_t *dbg_bins;     // nullable [B*Hq][2]
};

struct SelectParams {
    DecodeGeom g;
    const uint16_t *dl;
    const int32_t *lmax;
    const int32_t *sel;
    int32_t *cnt;          // [B*Hq][NC]
    int32_t *idx;          // [B*Hq][ld]
};

struct AttendParams {
    DecodeGeom g;
    CacheView c;
    const float *q;        // [B*Hq][128] the queries (exact scores from c.kf16)
    const uint32_t *qnib;
    const uint8_t *qa;     // [B*Hq][128] the codes as the fp8 operand of the matrix-core key products
    const float4 *qpar;
    float klog;            // log2(e) / sqrt(D)
    float kbin;            // Top-p bins per score unit (the score pass's)
    // Top-p selection (select mode only)
    const uint16_t *dl;
    const int32_t *lmax;
    const int32_t *sel;
    const int32_t *order;  // [B*Hq] head (b * Hq + h) of each dispatch rank
    const int32_t *order_ctr;  // [2]: order_ctr[0] heads were classed dense (attention chunk by chunk)
    // partial results per (b, h, chunk)
    float *pm;             // [B*Hq][NCA] the chunk's reference score: the max of its attended
                           // tokens, or (full softmax) up to 8 / klog below it
    float *pl;             // [B*Hq][NCA] sum of weights
    float *po;             // [B*Hq][NCA][128] weighted value sums
};

struct MergeParams {
    DecodeGeom g;
    float klog;
    const float *pm, *pl, *po;
    const float *tm, *tl, *to;  // nullable: the tail's partial (max score, weight sum, value sums)
    float *out;            // [B*Hq][128]
    int has_mass;          // accumulate attention mass (high-precision tier)
    MassParams mass;
};

// Exact attention over the binary16 tail: one partial (m, l, o) per (sequence, query head).

hipError_t launch_append(const AppendParams &p, hipStream_t s);
// Blocks of 256 threads with which the query-preparation launch can encode these new tokens
// (the randomized Hadamard rotation, or the dense one for at most 8192 token-heads), else 0.
long fused_append_blocks(const AppendParams &p);
hipError_t launch_qprep(const QprepParams &p, hipStream_t s);
hipError_t launch_score(const ScoreParams &p, hipStream_t s);
hipError_t launch_bin_scores(const BinScoresParams &p, hipStream_t s);
hipError_t launch_hist(const HistParams &p, hipStream_t s);
hipError_t launch_select(const SelectParams &p, hipStream_t s);
hipError_t launch_attend(const AttendParams &p, bool select, hipStream_t s);
hipError_t launch_merge(const MergeParams &p, hipStream_t s);

// Tail maintenance: append new tokens (binary16) / retire the first n tokens.
struct TailEditParams {
    uint16_t *k, *v;       // [B][cap][Hkv][128]
    int32_t *len;          // [B]
    int cap, Hkv, B;
    int dtype;             // append: 0 f16, 1 f32
    const void *nk, *nv;   // append: [B][n][Hkv][128]
    int n;                 // append: n_new; retire: n
    int32_t *seq_lens;     // retire: nullable
    float *mass;           // nullable [B][cap][Hkv]: zeroed for appended tokens, moved on retire
};
hipError_t launch_tail_append(const TailEditParams &p, hipStream_t s);
hipError_t launch_tail_retire(const TailEditParams &p, hipStream_t s);

// Promotion step of the high-precision tier (one block per (KV head, sequence)).
struct HpUpdateParams {
    CacheView c;
    uint16_t *hk, *hv;     // [B][Hkv][hcap][128]
    int32_t *hpos;         // [B][Hkv][hcap]
    uint32_t *hsaved;      // [B][Hkv][hcap]
    float *hmass;          // [B][Hkv][hcap]
    int hcap;
    const uint16_t *tk, *tv;  // tail [B][tcap][Hkv][128]
    const float *tmass;    // [B][tcap][Hkv]
    int tcap;
    int B, n;
    const int32_t *seq_lens;
    const int32_t *page_table;
    int max_pages;
};
hipError_t launch_hp_update(const HpUpdateParams &p, hipStream_t s);

// Bytes of the static workspace of kv_decode_attend_noalloc (per device).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// Device address of the static workspace on the device of stream s (taken once per device).
hipError_t static_scratch(hipStream_t s, void **ptr);

// Device-side argument checker (KV_DEBUG=1): one block per sequence checks the token range a
// call would touch -- [0, seq_lens[b]) for a decode, [start_pos[b], start_pos[b] + n_new) for
// an append -- against its bound and the page table entries covering it against num_pages.
// The first failure is recorded in a 4-word flag (code, sequence, page index, value).
struct CheckParams {
    const int32_t *seq_lens;   // nullable: decode lengths [B]
    int max_seq_len;
    const int32_t *start_pos;  // nullable: append positions [B]
    int n_new;
    const int32_t *page_table; // [B][max_pages]
    int B, max_pages, logP, num_pages;
};
enum { kCheckOk = 0, kCheckLen = 1, kCheckStart = 2, kCheckPage = 3 };
// Clears the flag, runs the checker and copies the flag to flag_host (4 words) on stream s; the
// caller synchronizes s before reading it.
hipError_t launch_check(const CheckParams &p, int32_t *flag_host, hipStream_t s);

}  // namespace kvc
