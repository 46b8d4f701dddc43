// C ABI of libkvcompress: argument validation (host only, before any HIP call), the decode
// plan (chunk size, workspace layout) and the launch sequences.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kv_compress.h"
#include "kvc_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(KV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(long x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(long x)
{
    int r = 0;
    while ((1L << r) < x) ++r;
    return r;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------------------
// Decode plan
// ---------------------------------------------------------------------------------------
struct Plan {
    kvc::DecodeGeom g;
    bool topp;
    int nsplit, cps;
    int hist_fused;  // the histogram and threshold passes in one kernel (k_hist_thresh)
    size_t off_qpl, off_qa, off_qpar, off_lmax, off_dl, off_hist, off_sel, off_cnt, off_order, off_octr, off_pm, off_pl, off_po, off_tm, off_tl, off_to;
    size_t total;
};

// Largest attention chunk (tokens of one attention wave).
int chunk_cap(bool topp)
{
    return topp ? kvc::kTopPAttendChunk : kvc::kMaxFullChunk;
}

// Geometry.
//  Full softmax: chunks of CH tokens, the largest power of two in [64, 2048] that still
//  gives at least 4096 waves (16 per compute unit) over (chunk, KV-head group, sequence),
//  and at most 512 when each KV head has one query head (GB = 1: the vector-unit pass for
//  64-dim value groups, whose waves then carry at most 8 batches), as long as no more than
//  kMaxChunks chunks result; one attention wave per chunk (KA = 1).
//  Top-p: score chunks of 512 tokens (one wave, 8 tokens per lane); an attention wave
//  (one query head: Top-p keeps a few, head-specific tokens) covers KA = 2 score chunks.
void plan_geometry(Plan &pl, int B, int rows_per_seq, int max_len, bool topp, int GB)
{
    int CH, KA = 1;
    if (topp) {
        CH = kvc::kTopPChunk;
        KA = kvc::kTopPAttendChunk / CH;
    } else {
        CH = chunk_cap(false);
        const long units = (long)B * rows_per_seq;
        const int cap = GB == 1 ? 512 : CH;
        while (CH > 64 && (CH > cap || units * ((max_len + CH - 1) / CH) < 4096) &&
               (long)(CH >> 1) * kvc::kMaxChunks >= max_len)
            CH >>= 1;
    }
    pl.g.CH = CH;
    pl.g.logCH = ilog2(CH);
    pl.g.NC = (max_len + CH - 1) / CH;
    if (pl.g.NC < 1) pl.g.NC = 1;
    pl.g.ld = max_len;
    pl.g.KA = KA;
    pl.g.NCA = (pl.g.NC + KA - 1) / KA;
    // rows of whole attention chunks, so that a chunk's distance loads need no bound
    pl.g.Lpad = pl.g.NCA * KA * CH;
}

void plan_layout(Plan &pl, int BH)
{
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    const size_t NC = (size_t)pl.g.NC, NCA = (size_t)pl.g.NCA;
    pl.off_qpl = take((size_t)BH * 16 * 4);
    pl.off_qa = take((size_t)BH * 128);
    pl.off_qpar = take((size_t)BH * 16);
    pl.off_pm = take((size_t)BH * NCA * 4);
    pl.off_pl = take((size_t)BH * NCA * 4);
    pl.off_po = take((size_t)BH * NCA * 128 * 4);
    // the binary16 tail's partial per (sequence, query head) (kv_decode_attend_tail)
    pl.off_tm = take((size_t)BH * 4);
    pl.off_tl = take((size_t)BH * 4);
    pl.off_to = take((size_t)BH * 128 * 4);
    if (pl.topp) {
        // histogram splits: >= 512 blocks over (split, head, sequence); a split holds fewer
        // than 65536 tokens (16-bit partial counts) and at most 256 chunks (one per thread)
        int nsplit = (512 + BH - 1) / BH;
        const int min_split = (int)(((long)pl.g.Lpad + 65535) / 65536);
        if (nsplit < min_split) nsplit = min_split;
        if (nsplit > pl.g.NC) nsplit = pl.g.NC;
        if (nsplit < 1) nsplit = 1;
        int cps = (pl.g.NC + nsplit - 1) / nsplit;
        while (cps > 256 || (long)cps * pl.g.CH > 65535) {  // one chunk per histogram thread; u16 counts
            ++nsplit;
            cps = (pl.g.NC + nsplit - 1) / nsplit;
        }
        pl.nsplit = nsplit;
        pl.cps = cps;
        // one block per head counts all its tokens and thresholds them: when the heads alone
        // give at least 128 blocks and a head's score chunks fit one per thread
        pl.hist_fused = BH >= 128 && pl.g.NC <= 1024;
        pl.off_lmax = take((size_t)BH * NC * 4);
        pl.off_dl = take((size_t)BH * pl.g.Lpad * 2);
        pl.off_hist = take((size_t)BH * nsplit * 8192 * 2);
        pl.off_sel = take((size_t)BH * 4 * 4);
        pl.off_cnt = take((size_t)BH * NC * 4);
        pl.off_order = take((size_t)BH * 4);
        pl.off_octr = take(2 * 4);
    } else {
        pl.nsplit = pl.cps = pl.hist_fused = 0;
        pl.off_lmax = pl.off_dl = pl.off_hist = pl.off_sel = pl.off_cnt = pl.off_order = pl.off_octr = 0;
    }
    pl.total = o;
}

int check_decode_shapes(int B, int Hq, int Hkv, int max_seq_len, int head_dim, float top_p)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_seq_len <= 0)
        return fail(KV_ERR_ARG, "B, Hq, Hkv and max_seq_len must be positive (got %d, %d, %d, %d)", B, Hq,
                    Hkv, max_seq_len);
    if (head_dim != 128) return fail(KV_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported", head_dim);
    if (Hq % Hkv != 0) return fail(KV_ERR_ARG, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(KV_ERR_UNSUPPORTED, "GQA group Hq/Hkv = %d: supported groups are 1, 2, 4, 8", G);
    if (!(top_p > 0.0f)) return fail(KV_ERR_ARG, "top_p must be > 0 (got %g)", (double)top_p);
    const long limit = (long)chunk_cap(top_p < 1.0f) * kvc::kMaxChunks;  // merge weights fit in LDS
    if (max_seq_len > limit)
        return fail(KV_ERR_UNSUPPORTED, "max_seq_len %d above %ld", max_seq_len, limit);
    if (B > 65535 || Hq > 65535)  // grid dimensions: sequences in z, query heads (or KV groups) in y
        return fail(KV_ERR_UNSUPPORTED, "B = %d, Hq = %d: at most 65535 sequences and query heads", B, Hq);
    return KV_OK;
}

void make_plan(Plan &pl, int B, int Hq, int Hkv, int max_seq_len, float top_p)
{
    memset(&pl, 0, sizeof(pl));
    pl.topp = top_p < 1.0f;
    const int G = Hq / Hkv;
    const int GB = G < 4 ? G : 4;
    pl.g.B = B;
    pl.g.Hq = Hq;
    pl.g.Hkv = Hkv;
    pl.g.G = G;
    pl.g.GB = GB;
    pl.g.nsub = G / GB;
    plan_geometry(pl, B, Hkv * pl.g.nsub, max_seq_len, pl.topp, GB);
    plan_layout(pl, B * Hq);
}

int check_cache(const kv_cache *c)
{
    if (!c) return fail(KV_ERR_ARG, "cache descriptor is NULL");
    if (c->head_dim != 128) return fail(KV_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported", c->head_dim);
    if (c->num_kv_heads <= 0) return fail(KV_ERR_ARG, "num_kv_heads must be positive");
    if (c->value_group != 32 && c->value_group != 64)
        return fail(KV_ERR_UNSUPPORTED, "value_group %d: supported groups are 32 and 64", c->value_group);
    if (!is_pow2(c->page_size) || c->page_size < 16)
        return fail(KV_ERR_UNSUPPORTED, "page_size %d: must be a power of two >= 16", c->page_size);
    if (c->num_pages <= 0) return fail(KV_ERR_ARG, "num_pages must be positive");
    if ((long)c->num_pages * c->num_kv_heads * c->page_size > 0xFFFFFFFFL)
        return fail(KV_ERR_UNSUPPORTED, "num_pages * num_kv_heads * page_size above 2^32 - 1 slots");
    if (c->rot_kind != KV_ROT_DENSE && c->rot_kind != KV_ROT_HADAMARD)
        return fail(KV_ERR_ARG, "rot_kind %d is not KV_ROT_DENSE or KV_ROT_HADAMARD", c->rot_kind);
    if (!c->rot || !c->keys || !c->vals)
        return fail(KV_ERR_ARG, "cache descriptor has a NULL array");
    if (c->keys_f16 && ((uintptr_t)c->keys_f16 & 15u) != 0)
        return fail(KV_ERR_ARG, "keys_f16 must be 16-byte aligned");
    if (c->key_center && ((uintptr_t)c->key_center & 15u) != 0)
        return fail(KV_ERR_ARG, "key_center must be 16-byte aligned");
    if (c->sketch_dim != 0 && c->sketch_dim != 128 && c->sketch_dim != 64)
        return fail(KV_ERR_UNSUPPORTED, "sketch_dim %d: supported widths are 128 (or 0) and 64", c->sketch_dim);
    return KV_OK;
}

int check_tail(const kv_tail *t, int32_t num_kv_heads, int32_t head_dim, int32_t B)
{
    if (!t) return fail(KV_ERR_ARG, "tail descriptor is NULL");
    if (!t->k || !t->v || !t->len) return fail(KV_ERR_ARG, "tail has a NULL array");
    if (t->capacity <= 0) return fail(KV_ERR_ARG, "tail capacity must be positive (got %d)", t->capacity);
    if ((((uintptr_t)t->k | (uintptr_t)t->v) & 15u) != 0) return fail(KV_ERR_ARG, "tail k and v must be 16-byte aligned");
    if (head_dim != 128) return fail(KV_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported", head_dim);
    if (num_kv_heads <= 0 || B <= 0) return fail(KV_ERR_ARG, "num_kv_heads and B must be positive");
    return KV_OK;
}

int check_hp(const kv_hp *hp)
{
    if (!hp->k || !hp->v || !hp->pos || !hp->saved || !hp->mass) return fail(KV_ERR_ARG, "tier has a NULL array");
    if (hp->capacity <= 0 || hp->capacity > 1024)
        return fail(KV_ERR_ARG, "tier capacity must be in 1..1024 (got %d)", hp->capacity);
    if ((((uintptr_t)hp->k | (uintptr_t)hp->v) & 15u) != 0) return fail(KV_ERR_ARG, "tier k and v must be 16-byte aligned");
    if ((((uintptr_t)hp->pos | (uintptr_t)hp->saved | (uintptr_t)hp->mass) & 3u) != 0)
        return fail(KV_ERR_ARG, "tier pos, saved and mass must be 4-byte aligned");
    return KV_OK;
}

kvc::CacheView view_of(const kv_cache *c)
{
    kvc::CacheView v;
    v.Hkv = c->num_kv_heads;
    v.P = c->page_size;
    v.logP = ilog2(c->page_size);
    v.Gv = c->value_group;
    v.lngrp = ilog2(c->head_dim / c->value_group);
    v.keys = c->keys;
    v.vals = c->vals;
    v.kf16 = c->keys_f16;
    v.kc = c->key_center;
    v.sk = c->sketch_dim == 0 ? c->head_dim : c->sketch_dim;
    v.kw = v.sk / 32;
    return v;
}

// Stage events, when the caller asked for them: the stage's kernels record them as they
// begin and end (hipExtLaunchKernel, see kvc::StageTiming).
void stage_mark(const kv_debug *dbg, int stage, bool begin, hipStream_t)
{
    if (!dbg || !dbg->stage_events) return;
    if (begin) kvc::g_stage_timing = {dbg->stage_events[2 * stage], dbg->stage_events[2 * stage + 1]};
    else kvc::g_stage_timing = {nullptr, nullptr};
}

template <typename T>
T *at(void *ws, size_t off)
{
    return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

// KV_DEBUG=1 (read at every call): device-side argument checks before a call enqueues its
// kernels.  The checker reads seq_lens / start_pos and the page table entries the call would
// use, the stream is synchronized, and a failure becomes KV_ERR_ARG.
bool debug_checks()
{
    const char *v = getenv("KV_DEBUG");
    return v && v[0] == '1' && v[1] == 0;
}

int run_check(const kvc::CheckParams &p, hipStream_t stream)
{
    int32_t flag[4] = {0, 0, 0, 0};
    hipError_t e = kvc::launch_check(p, flag, stream);
    if (e != hipSuccess) return hip_fail(e, "argument checker");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "argument checker synchronize");
    switch (flag[0]) {
    case kvc::kCheckOk: return KV_OK;
    case kvc::kCheckLen:
        return fail(KV_ERR_ARG, "KV_DEBUG: seq_lens[%d] = %d is outside 0..max_seq_len (%d)", flag[1], flag[3],
                    p.max_seq_len);
    case kvc::kCheckStart:
        return fail(KV_ERR_ARG, "KV_DEBUG: start_pos[%d] = %d: the %d new tokens leave the %d mapped pages", flag[1],
                    flag[3], p.n_new, p.max_pages);
    default:
        return fail(KV_ERR_ARG, "KV_DEBUG: page_table[%d][%d] = %d is outside 0..num_pages-1 (%d pages)", flag[1],
                    flag[2], flag[3], p.num_pages);
    }
}

// Checks of a decode (seq_lens) or an append (start_pos, n_new) against the page table.
int check_on_device(const kv_cache *c, const int32_t *seq_lens, int max_seq_len, const int32_t *start_pos,
                    int n_new, const int32_t *page_table, int B, int max_pages, hipStream_t stream)
{
    kvc::CheckParams p;
    p.seq_lens = seq_lens;
    p.max_seq_len = max_seq_len;
    p.start_pos = start_pos;
    p.n_new = n_new;
    p.page_table = page_table;
    p.B = B;
    p.max_pages = max_pages;
    p.logP = ilog2(c->page_size);
    p.num_pages = c->num_pages;
    return run_check(p, stream);
}

}  // namespace

extern "C" {

const char *kv_last_error(void) { return g_err; }

int kv_version(void) { return 10000; }

}  // extern "C"

namespace {

// Checks the arguments of an append (the cache already checked) and fills its parameters;
// n_new == 0 gives KV_OK with p.n_new = 0.
int make_append(const kv_cache *c, int32_t dtype, const void *k, const void *v, int32_t B, int32_t n_new,
                const int32_t *start_pos, const int32_t *page_table, int32_t max_pages, kvc::AppendParams &p)
{
    if (dtype != KV_F16 && dtype != KV_F32) return fail(KV_ERR_ARG, "dtype %d is not KV_F16 or KV_F32", dtype);
    if (B <= 0 || n_new < 0 || max_pages <= 0)
        return fail(KV_ERR_ARG, "B and max_pages must be positive and n_new >= 0 (got %d, %d, %d)", B, n_new,
                    max_pages);
    p.n_new = 0;
    if (n_new == 0) return KV_OK;
    if (!k || !v || !start_pos || !page_table) return fail(KV_ERR_ARG, "NULL k, v, start_pos or page_table");
    p.c = view_of(c);
    p.rot_kind = c->rot_kind;
    p.rot = c->rot;
    p.dtype = dtype;
    p.k = k;
    p.v = v;
    p.B = B;
    p.n_new = n_new;
    p.start_pos = start_pos;
    p.page_table = page_table;
    p.max_pages = max_pages;
    return KV_OK;
}

}  // namespace

extern "C" {

int kv_compress_append(const kv_cache *c, int32_t dtype, const void *k, const void *v, int32_t B,
                       int32_t n_new, const int32_t *start_pos, const int32_t *page_table,
                       int32_t max_pages, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_cache(c);
    if (rc) return rc;
    kvc::AppendParams p;
    rc = make_append(c, dtype, k, v, B, n_new, start_pos, page_table, max_pages, p);
    if (rc || p.n_new == 0) return rc;
    if (debug_checks()) {
        rc = check_on_device(c, nullptr, 0, start_pos, n_new, page_table, B, max_pages, stream);
        if (rc) return rc;
    }
    hipError_t e = kvc::launch_append(p, stream);
    if (e != hipSuccess) return hip_fail(e, "append launch");
    return KV_OK;
}

size_t kv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len, int32_t head_dim,
                                 float top_p)
{
    if (check_decode_shapes(B, Hq, Hkv, max_seq_len, head_dim, top_p) != KV_OK) return 0;
    Plan pl;
    make_plan(pl, B, Hq, Hkv, max_seq_len, top_p);
    return pl.total;
}

size_t kv_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_seq_len, int32_t head_dim, float top_p)
{
    return kv_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, head_dim, top_p);
}

namespace {

int decode_impl(const kv_cache *c, const kv_tail *tail, const kv_hp *hp, const float *dither,
                const kv_append_args *app, const float *q, int32_t B, int32_t Hq,
                const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table, int32_t max_pages,
                float top_p, float *out, const kv_debug *dbg, void *workspace, size_t workspace_bytes,
                hipStream_t stream)
{
    struct TimingGuard {  // no stage timing outlives the call, whatever path it returns by
        ~TimingGuard() { kvc::g_stage_timing = {nullptr, nullptr}; }
    } timing_guard;
    int rc = check_cache(c);
    if (rc) return rc;
    rc = check_decode_shapes(B, Hq, c->num_kv_heads, max_seq_len, c->head_dim, top_p);
    if (rc) return rc;
    if (!q || !seq_lens || !page_table || !out) return fail(KV_ERR_ARG, "NULL q, seq_lens, page_table or out");
    if (max_pages <= 0) return fail(KV_ERR_ARG, "max_pages must be positive");
    if ((long)max_pages * c->page_size < (long)max_seq_len)
        return fail(KV_ERR_ARG, "max_pages * page_size (%ld) < max_seq_len (%d)", (long)max_pages * c->page_size,
                    max_seq_len);
    Plan pl;
    make_plan(pl, B, Hq, c->num_kv_heads, max_seq_len, top_p);
    if (!workspace || workspace_bytes < pl.total)
        return fail(KV_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes required", workspace_bytes,
                    pl.total);
    pl.g.seq_lens = seq_lens;
    pl.g.page_table = page_table;
    pl.g.max_pages = max_pages;
    if (debug_checks()) {
        if (app && app->n_new > 0 && app->start_pos) {
            rc = check_on_device(c, nullptr, 0, app->start_pos, app->n_new, page_table, B, max_pages, stream);
            if (rc) return rc;
        }
        rc = check_on_device(c, seq_lens, max_seq_len, nullptr, 0, page_table, B, max_pages, stream);
        if (rc) return rc;
    }
    const kvc::CacheView cv = view_of(c);
    const float isd = (float)(1.0 / sqrt((double)c->head_dim));
    const float kbin = (float)(256.0 * 1.4426950408889634074 / sqrt((double)c->head_dim));
    const float klog = (float)(1.4426950408889634074 / sqrt((double)c->head_dim));
    (void)isd;
    const int BH = B * Hq;
    uint32_t *qnib = at<uint32_t>(workspace, pl.off_qpl);
    float4 *qpar = at<float4>(workspace, pl.off_qpar);
    uint8_t *qa = at<uint8_t>(workspace, pl.off_qa);

    kvc::QprepParams qp;
    qp.rot_kind = c->rot_kind;
    qp.rot = c->rot;
    qp.q = q;
    qp.BH = BH;
    qp.qnib = qnib;
    qp.qa = qa;
    qp.qpar = qpar;
    qp.dbg_codes = dbg ? dbg->q_codes : nullptr;
    qp.dbg_params = dbg ? dbg->q_params : nullptr;
    qp.dbg_sumu = dbg ? dbg->q_sumu : nullptr;
    qp.sk = cv.sk;
    qp.isk = (float)(1.0 / sqrt((double)cv.sk));
    qp.dither = dither;
    qp.app_blocks = 0;
    qp.app_N = 0;
    qp.order_ctr = pl.topp ? at<int32_t>(workspace, pl.off_octr) : nullptr;
    if (app) {
        rc = make_append(c, app->dtype, app->k, app->v, B, app->n_new, app->start_pos, page_table, max_pages, qp.app);
        if (rc) return rc;
        if (qp.app.n_new > 0) {
            qp.app_blocks = kvc::fused_append_blocks(qp.app);
            qp.app_N = (long)B * qp.app.n_new * c->num_kv_heads;
            if (qp.app_blocks == 0) {  // too many tokens to ride along: an append launch first
                hipError_t ea = kvc::launch_append(qp.app, stream);
                if (ea != hipSuccess) return hip_fail(ea, "append launch");
            }
        }
    }
    qp.has_tail = tail != nullptr || hp != nullptr;
    if (qp.has_tail) {
        kvc::TailParams &tp = qp.tail;
        tp.B = B;
        tp.Hq = Hq;
        tp.G = Hq / c->num_kv_heads;
        tp.Hkv = c->num_kv_heads;
        tp.klog = klog;
        tp.q = q;
        tp.k = tail ? tail->k : nullptr;
        tp.v = tail ? tail->v : nullptr;
        tp.len = tail ? tail->len : nullptr;
        tp.cap = tail ? tail->capacity : 0;
        tp.hk = hp ? hp->k : nullptr;
        tp.hv = hp ? hp->v : nullptr;
        tp.hpos = hp ? hp->pos : nullptr;
        tp.hcap = hp ? hp->capacity : 0;
        tp.tm = at<float>(workspace, pl.off_tm);
        tp.tl = at<float>(workspace, pl.off_tl);
        tp.to = at<float>(workspace, pl.off_to);
        // exact scores of the compressed tokens (binary16 keys under Top-p) are uncentered
        tp.center = (c->keys_f16 && pl.topp) ? nullptr : c->key_center;
    }
    stage_mark(dbg, KV_STAGE_QUERY, true, stream);
    hipError_t e = kvc::launch_qprep(qp, stream);
    if (e != hipSuccess) return hip_fail(e, "query launch");
    stage_mark(dbg, KV_STAGE_QUERY, false, stream);

    kvc::ScoreParams sp;
    sp.g = pl.g;
    sp.c = cv;
    sp.qnib = qnib;
    sp.qa = qa;
    sp.qpar = qpar;
    sp.kbin = kbin;
    sp.dl = pl.topp ? at<uint16_t>(workspace, pl.off_dl) : nullptr;
    sp.lmax = pl.topp ? at<int32_t>(workspace, pl.off_lmax) : nullptr;
    sp.dbg_scores = dbg ? dbg->scores : nullptr;
    sp.dbg_iscores = dbg ? dbg->iscores : nullptr;
    if (pl.topp || sp.dbg_scores || sp.dbg_iscores) {
        stage_mark(dbg, KV_STAGE_SCORE, true, stream);
        e = kvc::launch_score(sp, stream);
        if (e != hipSuccess) return hip_fail(e, "score launch");
        stage_mark(dbg, KV_STAGE_SCORE, false, stream);
    }
    if (pl.topp && dbg && dbg->bin_dist) {  // what the score pass wrote, row by row
        e = hipMemcpy2DAsync(dbg->bin_dist, (size_t)pl.g.ld * 2, sp.dl, (size_t)pl.g.Lpad * 2, (size_t)pl.g.ld * 2,
                             (size_t)BH, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "bin distance copy");
    }
    if (pl.topp && dbg && dbg->chunk_top) {
        e = hipMemcpyAsync(dbg->chunk_top, sp.lmax, (size_t)BH * pl.g.NC * 4, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "chunk top copy");
    }

    if (pl.topp) {
        kvc::HistParams hp;
        hp.g = pl.g;
        hp.nsplit = pl.nsplit;
        hp.cps = pl.cps;
        hp.fused = pl.hist_fused;
        hp.pfx = (uint32_t)rint((double)top_p * 16777216.0);
        hp.dl = sp.dl;
        hp.lmax = sp.lmax;
        hp.hist = at<uint16_t>(workspace, pl.off_hist);
        hp.sel = at<int32_t>(workspace, pl.off_sel);
        hp.order = at<int32_t>(workspace, pl.off_order);
        hp.order_ctr = at<int32_t>(workspace, pl.off_octr);
        hp.dbg_count = dbg ? dbg->sel_count : nullptr;
        hp.dbg_bins = dbg ? dbg->sel_bins : nullptr;
        stage_mark(dbg, KV_STAGE_HIST, true, stream);
        e = kvc::launch_hist(hp, stream);
        if (e != hipSuccess) return hip_fail(e, "histogram launch");
        stage_mark(dbg, KV_STAGE_HIST, false, stream);
        if (dbg && dbg->sel_idx) {
            kvc::SelectParams sel;
            sel.g = pl.g;
            sel.dl = sp.dl;
            sel.lmax = sp.lmax;
            sel.sel = hp.sel;
            sel.cnt = at<int32_t>(workspace, pl.off_cnt);
            sel.idx = dbg->sel_idx;
            stage_mark(dbg, KV_STAGE_SELECT, true, stream);
            e = kvc::launch_select(sel, stream);
            if (e != hipSuccess) return hip_fail(e, "selection launch");
            stage_mark(dbg, KV_STAGE_SELECT, false, stream);
        }
    }

    kvc::AttendParams ap;
    ap.g = pl.g;
    ap.c = cv;
    ap.q = q;
    ap.qnib = qnib;
    ap.qa = qa;
    ap.qpar = qpar;
    ap.klog = klog;
    ap.kbin = kbin;
    ap.dl = sp.dl;
    ap.lmax = sp.lmax;
    ap.sel = pl.topp ? at<int32_t>(workspace, pl.off_sel) : nullptr;
    ap.order = pl.topp ? at<int32_t>(workspace, pl.off_order) : nullptr;
    ap.order_ctr = pl.topp ? at<int32_t>(workspace, pl.off_octr) : nullptr;
    ap.pm = at<float>(workspace, pl.off_pm);
    ap.pl = at<float>(workspace, pl.off_pl);
    ap.po = at<float>(workspace, pl.off_po);
    stage_mark(dbg, KV_STAGE_ATTEND, true, stream);
    e = kvc::launch_attend(ap, pl.topp, stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    stage_mark(dbg, KV_STAGE_ATTEND, false, stream);

    kvc::MergeParams mp;
    mp.g = pl.g;
    mp.klog = klog;
    mp.pm = ap.pm;
    mp.pl = ap.pl;
    mp.po = ap.po;
    mp.tm = mp.tl = mp.to = nullptr;
    mp.out = out;
    mp.has_mass = 0;
    if (qp.has_tail) {
        mp.tm = qp.tail.tm;
        mp.tl = qp.tail.tl;
        mp.to = qp.tail.to;
    }
    if (hp) {
        kvc::MassParams &ms = mp.mass;
        mp.has_mass = 1;
        ms.q = q;
        ms.center = qp.tail.center;
        ms.tk = tail ? tail->k : nullptr;
        ms.tlen = tail ? tail->len : nullptr;
        ms.tcap = tail ? tail->capacity : 0;
        ms.tmass = tail ? tail->mass : nullptr;
        ms.hk = hp->k;
        ms.hpos = hp->pos;
        ms.hmass = hp->mass;
        ms.hcap = hp->capacity;
    }
    stage_mark(dbg, KV_STAGE_MERGE, true, stream);
    e = kvc::launch_merge(mp, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    stage_mark(dbg, KV_STAGE_MERGE, false, stream);
    return KV_OK;
}

}  // namespace

int kv_decode_attend(const kv_cache *c, const float *q, int32_t B, int32_t Hq, const int32_t *seq_lens,
                     int32_t max_seq_len, const int32_t *page_table, int32_t max_pages, float top_p,
                     float *out, const kv_debug *dbg, void *workspace, size_t workspace_bytes,
                     hipStream_t stream)
{
    g_err[0] = 0;
    return decode_impl(c, nullptr, nullptr, nullptr, nullptr, q, B, Hq, seq_lens, max_seq_len, page_table, max_pages,
                       top_p, out, dbg, workspace, workspace_bytes, stream);
}

int kv_decode_attend_tail(const kv_cache *c, const kv_tail *tail, const float *q, int32_t B, int32_t Hq,
                          const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                          int32_t max_pages, float top_p, float *out, const kv_debug *dbg, void *workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    if (!c) return fail(KV_ERR_ARG, "cache descriptor is NULL");
    int rc = check_tail(tail, c->num_kv_heads, c->head_dim, B);
    if (rc) return rc;
    return decode_impl(c, tail, nullptr, nullptr, nullptr, q, B, Hq, seq_lens, max_seq_len, page_table, max_pages,
                       top_p, out, dbg, workspace, workspace_bytes, stream);
}

namespace {

int decode_ex(const kv_cache *c, const kv_decode_opts *opts, const float *q, int32_t B, int32_t Hq,
              const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table, int32_t max_pages, float top_p,
              float *out, const kv_debug *dbg, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!c) return fail(KV_ERR_ARG, "cache descriptor is NULL");
    const kv_tail *tail = opts ? opts->tail : nullptr;
    const float *dither = opts ? opts->q_dither : nullptr;
    const kv_hp *hp = opts ? opts->hp : nullptr;
    if (tail) {
        int rc = check_tail(tail, c->num_kv_heads, c->head_dim, B);
        if (rc) return rc;
    }
    if (hp) {
        int rc = check_hp(hp);
        if (rc) return rc;
        if (tail && !tail->mass) return fail(KV_ERR_ARG, "a tier with a tail needs the tail's mass array");
    }
    if (dither && ((uintptr_t)dither & 3u) != 0) return fail(KV_ERR_ARG, "q_dither must be 4-byte aligned");
    const kv_append_args *app = opts ? opts->append : nullptr;
    return decode_impl(c, tail, hp, dither, app, q, B, Hq, seq_lens, max_seq_len, page_table, max_pages, top_p, out,
                       dbg, workspace, workspace_bytes, stream);
}

}  // namespace

int kv_decode_attend_ex(const kv_cache *c, const kv_decode_opts *opts, const float *q, int32_t B, int32_t Hq,
                        const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                        int32_t max_pages, float top_p, float *out, const kv_debug *dbg, void *workspace,
                        size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    return decode_ex(c, opts, q, B, Hq, seq_lens, max_seq_len, page_table, max_pages, top_p, out, dbg, workspace,
                     workspace_bytes, stream);
}

int kv_decode_attend_noalloc(const kv_cache *c, const kv_decode_opts *opts, const float *q, int32_t B, int32_t Hq,
                             const int32_t *seq_lens, int32_t max_seq_len, const int32_t *page_table,
                             int32_t max_pages, float top_p, float *out, const kv_debug *dbg, hipStream_t stream)
{
    g_err[0] = 0;
    if (!c) return fail(KV_ERR_ARG, "cache descriptor is NULL");
    int rc = check_decode_shapes(B, Hq, c->num_kv_heads, max_seq_len, c->head_dim, top_p);
    if (rc) return rc;
    Plan pl;
    make_plan(pl, B, Hq, c->num_kv_heads, max_seq_len, top_p);
    if (pl.total > kvc::kStaticScratchBytes)
        return fail(KV_ERR_WORKSPACE,
                    "this decode needs %zu bytes of workspace, above the %zu bytes of the static workspace of "
                    "kv_decode_attend_noalloc (use kv_decode_attend_ex with a caller workspace)",
                    pl.total, kvc::kStaticScratchBytes);
    void *ws = nullptr;
    hipError_t e = kvc::static_scratch(stream, &ws);
    if (e != hipSuccess) return hip_fail(e, "static workspace address");
    return decode_ex(c, opts, q, B, Hq, seq_lens, max_seq_len, page_table, max_pages, top_p, out, dbg, ws, pl.total,
                     stream);
}

int kv_hp_update(const kv_cache *c, const kv_hp *hp, const kv_tail *t, int32_t B, int32_t n,
                 const int32_t *seq_lens, const int32_t *page_table, int32_t max_pages, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_cache(c);
    if (rc) return rc;
    if (!hp) return fail(KV_ERR_ARG, "tier descriptor is NULL");
    rc = check_hp(hp);
    if (rc) return rc;
    rc = check_tail(t, c->num_kv_heads, c->head_dim, B);
    if (rc) return rc;
    if (!t->mass) return fail(KV_ERR_ARG, "the tail has no mass array");
    if (n < 0 || n > t->capacity) return fail(KV_ERR_ARG, "n must be in 0..tail capacity (got %d)", n);
    if (hp->capacity + n > 1024) return fail(KV_ERR_ARG, "tier capacity + n must be <= 1024");
    if (!seq_lens || !page_table) return fail(KV_ERR_ARG, "NULL seq_lens or page_table");
    if (max_pages <= 0) return fail(KV_ERR_ARG, "max_pages must be positive");
    if (n == 0) return KV_OK;
    kvc::HpUpdateParams p;
    p.c = view_of(c);
    p.hk = hp->k;
    p.hv = hp->v;
    p.hpos = hp->pos;
    p.hsaved = hp->saved;
    p.hmass = hp->mass;
    p.hcap = hp->capacity;
    p.tk = t->k;
    p.tv = t->v;
    p.tmass = t->mass;
    p.tcap = t->capacity;
    p.B = B;
    p.n = n;
    p.seq_lens = seq_lens;
    p.page_table = page_table;
    p.max_pages = max_pages;
    hipError_t e = kvc::launch_hp_update(p, stream);
    return e == hipSuccess ? KV_OK : hip_fail(e, "tier update launch");
}

int kv_tail_append(const kv_tail *t, int32_t num_kv_heads, int32_t head_dim, int32_t dtype, const void *k,
                   const void *v, int32_t B, int32_t n_new, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_tail(t, num_kv_heads, head_dim, B);
    if (rc) return rc;
    if (dtype != KV_F16 && dtype != KV_F32) return fail(KV_ERR_ARG, "dtype %d is not KV_F16 or KV_F32", dtype);
    if (n_new < 0) return fail(KV_ERR_ARG, "n_new must be >= 0 (got %d)", n_new);
    if (n_new == 0) return KV_OK;
    if (!k || !v) return fail(KV_ERR_ARG, "NULL k or v");
    kvc::TailEditParams p;
    p.k = t->k;
    p.v = t->v;
    p.len = t->len;
    p.cap = t->capacity;
    p.Hkv = num_kv_heads;
    p.B = B;
    p.dtype = dtype;
    p.nk = k;
    p.nv = v;
    p.n = n_new;
    p.seq_lens = nullptr;
    p.mass = t->mass;
    hipError_t e = kvc::launch_tail_append(p, stream);
    return e == hipSuccess ? KV_OK : hip_fail(e, "tail append launch");
}

int kv_tail_retire(const kv_tail *t, int32_t num_kv_heads, int32_t head_dim, int32_t B, int32_t n,
                   int32_t *seq_lens, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_tail(t, num_kv_heads, head_dim, B);
    if (rc) return rc;
    if (n < 0) return fail(KV_ERR_ARG, "n must be >= 0 (got %d)", n);
    if (n == 0) return KV_OK;
    kvc::TailEditParams p;
    p.k = t->k;
    p.v = t->v;
    p.len = t->len;
    p.cap = t->capacity;
    p.Hkv = num_kv_heads;
    p.B = B;
    p.dtype = 0;
    p.nk = p.nv = nullptr;
    p.n = n;
    p.seq_lens = seq_lens;
    p.mass = t->mass;
    hipError_t e = kvc::launch_tail_retire(p, stream);
    return e == hipSuccess ? KV_OK : hip_fail(e, "tail retire launch");
}

size_t kv_topp_workspace_bytes(int32_t B, int32_t Hq, int32_t ld)
{
    if (B <= 0 || Hq <= 0 || ld <= 0 || ld > (1 << 30)) return 0;
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.topp = true;
    pl.g.B = B;
    pl.g.Hq = Hq;
    pl.g.Hkv = Hq;
    pl.g.G = pl.g.GB = pl.g.nsub = 1;
    plan_geometry(pl, B, Hq, ld, true, 1);
    plan_layout(pl, B * Hq);
    return pl.total;
}

int kv_topp_select(const float *scores, int32_t ld, const int32_t *seq_lens, int32_t B, int32_t Hq,
                   int32_t head_dim, float top_p, int32_t *sel_idx, int32_t *sel_count, void *workspace,
                   size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    if (B <= 0 || Hq <= 0 || ld <= 0)
        return fail(KV_ERR_ARG, "B, Hq and ld must be positive (got %d, %d, %d)", B, Hq, ld);
    if (ld > (1 << 30)) return fail(KV_ERR_UNSUPPORTED, "ld %d above 2^30", ld);
    if (head_dim <= 0) return fail(KV_ERR_ARG, "head_dim must be positive");
    if (!(top_p > 0.0f && top_p < 1.0f)) return fail(KV_ERR_ARG, "top_p must be in (0, 1) (got %g)", (double)top_p);
    if (!scores || !seq_lens || !sel_idx || !sel_count)
        return fail(KV_ERR_ARG, "NULL scores, seq_lens, sel_idx or sel_count");
    const size_t need = kv_topp_workspace_bytes(B, Hq, ld);
    if (!workspace || workspace_bytes < need)
        return fail(KV_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu bytes required", workspace_bytes,
                    need);
    Plan pl;
    memset(&pl, 0, sizeof(pl));
    pl.topp = true;
    pl.g.B = B;
    pl.g.Hq = Hq;
    pl.g.Hkv = Hq;
    pl.g.G = pl.g.GB = pl.g.nsub = 1;
    plan_geometry(pl, B, Hq, ld, true, 1);
    plan_layout(pl, B * Hq);
    pl.g.seq_lens = seq_lens;
    pl.g.page_table = nullptr;
    pl.g.max_pages = 0;
    const float kbin = (float)(256.0 * 1.4426950408889634074 / sqrt((double)head_dim));

    kvc::BinScoresParams bp;
    bp.g = pl.g;
    bp.scores = scores;
    bp.kbin = kbin;
    bp.dl = at<uint16_t>(workspace, pl.off_dl);
    bp.lmax = at<int32_t>(workspace, pl.off_lmax);
    hipError_t e = kvc::launch_bin_scores(bp, stream);
    if (e != hipSuccess) return hip_fail(e, "bin launch");
    kvc::HistParams hp;
    hp.g = pl.g;
    hp.nsplit = pl.nsplit;
    hp.cps = pl.cps;
    hp.fused = pl.hist_fused;
    hp.pfx = (uint32_t)rint((double)top_p * 16777216.0);
    hp.dl = bp.dl;
    hp.lmax = bp.lmax;
    hp.hist = at<uint16_t>(workspace, pl.off_hist);
    hp.sel = at<int32_t>(workspace, pl.off_sel);
    hp.order = hp.order_ctr = nullptr;
    hp.dbg_count = sel_count;
    hp.dbg_bins = nullptr;
    e = kvc::launch_hist(hp, stream);
    if (e != hipSuccess) return hip_fail(e, "histogram launch");
    kvc::SelectParams sel;
    sel.g = pl.g;
    sel.dl = bp.dl;
    sel.lmax = bp.lmax;
    sel.sel = hp.sel;
    sel.cnt = at<int32_t>(workspace, pl.off_cnt);
    sel.idx = sel_idx;
    e = kvc::launch_select(sel, stream);
    if (e != hipSuccess) return hip_fail(e, "selection launch");
    return KV_OK;
}

}  // extern "C"
