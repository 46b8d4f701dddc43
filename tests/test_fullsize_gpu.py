"""Full-size parity on the workloads' real shapes, inputs drawn on the device by torch's
seeded generator:

- the 128k-context GQA Top-p workload (batch 4, 32 query / 8 KV heads, 131072 tokens, 1%
  spike tokens, Top-p 0.9) in the launch configuration the benchmark times;
- 32 sequences x 32 heads of lengths 1k..32k on shuffled 256-token pages, value group 64,
  full softmax;
- the 32768-token x 32-head prefill append with a randomized Hadamard rotation, then a
  1,048,576-token decode over 8 KV heads at Top-p 0.95 whose cache 32 appends built.

The oracle checks sampled (sequence, KV head) units one by one: the unit's cache bytes,
then the library's scores, Top-p sets and outputs for the unit's query heads.  Properties
that hold at any size are checked on every head.  The decode without score output (the
kernels the benchmark times) must give the same Top-p sets and bit-identical outputs as the
decode with score output."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads as W
from tests.kvc_testlib import Case, check_bins, chunk_dists, compare_caches, download, gpu_append, oracle_cache_of, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SAMPLED_UNITS = [(0, 0), (3, 7)]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_gqa_128k_topp_full_size():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc

    wl = W.CONFIGS[2]
    dev = torch.device("cuda")
    B, Hq, Hkv, L, G = wl.B, wl.Hq, wl.Hkv, wl.L, wl.Hq // wl.Hkv
    _say(f"[full] {wl.name}: drawing inputs")
    K, V, q = W.draw_device(wl, dev)
    lens = np.full(B, L, np.int32)
    pt_np, npages = W.page_layout(wl, lens)
    kind, R16 = W.draw_rotation(wl)
    cache = kvc.KVCache(npages, Hkv, R16, rot_kind=kind, page_size=wl.P, value_group=wl.Gv, device=dev)
    pt = torch.from_numpy(pt_np).to(dev)
    seq = torch.from_numpy(lens).to(dev)
    kvc.append(cache, K, V, torch.zeros(B, dtype=torch.int32, device=dev), pt)
    dbg = kvc.DecodeDebug.allocate(B, Hq, L, True, dev)
    out = kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=L, debug=dbg)
    out_full = kvc.decode_attend(cache, q, seq, pt, top_p=1.0, max_seq_len=L)
    # the decode as the benchmark runs it (no score output: the matrix-core score pass)
    dbg_fast = kvc.DecodeDebug.allocate(B, Hq, L, True, dev, scores=False, dist=True)
    out_fast = kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=L, debug=dbg_fast)
    torch.cuda.synchronize()
    _say("[full] library decode done")
    np.testing.assert_array_equal(dbg_fast.sel_count.cpu().numpy(), dbg.sel_count.cpu().numpy())
    np.testing.assert_array_equal(dbg_fast.sel_bins.cpu().numpy(), dbg.sel_bins.cpu().numpy())
    assert torch.equal(dbg_fast.sel_idx, dbg.sel_idx)
    assert torch.equal(out_fast.view(torch.int32), out.view(torch.int32))
    fast_dist = {u: (dbg_fast.bin_dist[u[0], u[1] * G:(u[1] + 1) * G].cpu().numpy().view(np.uint16),
                     dbg_fast.chunk_top[u[0], u[1] * G:(u[1] + 1) * G].cpu().numpy()) for u in SAMPLED_UNITS}
    del dbg_fast, out_fast

    # properties on every (sequence, query head)
    cnt = dbg.sel_count.cpu().numpy()
    assert np.all(cnt >= 1) and np.all(cnt <= L)
    idx = dbg.sel_idx.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            sel = idx[b, h, :cnt[b, h]]
            assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < L
    assert torch.isfinite(out).all() and torch.isfinite(out_full).all()

    # sampled units against the oracle
    orot = oracle.Rotation(oracle.ROT_DENSE, wl.D, R16=R16)
    qn = q.cpu().numpy()

    def unit(bh):
        b, h = bh
        k = K[b, :, h].float().cpu().numpy()
        v = V[b, :, h].float().cpu().numpy()
        bits, nc = oracle.key_encode(orot, k)
        codes, sz = oracle.value_encode(v, wl.D, wl.Gv)
        res = []
        for hh in range(h * G, (h + 1) * G):
            qe = oracle.query_encode(orot, qn[b, hh][None, :])
            _, _, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], wl.D)
            tp = oracle.topp(s, wl.top_p, wl.D)
            res.append(dict(s=s, tp=tp, out=oracle.attend(s, codes, sz, wl.D, wl.Gv, tp["idx"]),
                            out_full=oracle.attend(s, codes, sz, wl.D, wl.Gv)))
        return bits, nc, codes, sz, res

    with ThreadPoolExecutor(len(SAMPLED_UNITS)) as ex:
        refs = list(ex.map(unit, SAMPLED_UNITS))
    scores = dbg.scores
    kb = cache.key_bits.cpu().numpy().view(np.uint32)
    kn = cache.key_nc.cpu().numpy().view(np.uint32)
    vc = cache.val_codes.cpu().numpy()
    vs = cache.val_sz.cpu().numpy().view(np.uint32)
    o, of = out.cpu().numpy(), out_full.cpu().numpy()
    for (b, h), (bits, nc, codes, sz, res) in zip(SAMPLED_UNITS, refs):
        t = np.arange(L)
        pg, sl = pt_np[b, t // wl.P], t % wl.P
        np.testing.assert_array_equal(kb[pg, h, sl], bits)
        np.testing.assert_array_equal(kn[pg, h, sl] & 0xFFFF, nc[:, 0])
        assert np.all(np.abs((kn[pg, h, sl] >> 16).astype(np.int64) - nc[:, 1].astype(np.int64)) <= 1)
        np.testing.assert_array_equal(vc[pg, h, sl], codes)
        np.testing.assert_array_equal(vs[pg, h, sl], sz[..., 0].astype(np.uint32) | (sz[..., 1].astype(np.uint32) << 16))
        same = np.array_equal(kn[pg, h, sl] >> 16, nc[:, 1])
        # the oracle's scores and Top-p on the records the library wrote: compared always
        ncw = kn[pg, h, sl]
        nc_g = np.stack([(ncw & 0xFFFF).astype(np.uint16), (ncw >> 16).astype(np.uint16)], axis=-1)
        fd, ft = fast_dist[(b, h)]
        for j, hh in enumerate(range(h * G, (h + 1) * G)):
            r = res[j]
            qe = oracle.query_encode(orot, qn[b, hh][None, :])
            _, _, s_g = oracle.scores(kb[pg, h, sl], nc_g, qe["u"][0], qe["c0"][0], qe["c1"][0], wl.D)
            tp_g = oracle.topp(s_g, wl.top_p, wl.D)
            np.testing.assert_array_equal(scores[b, hh].cpu().numpy().view(np.uint32), s_g.view(np.uint32))
            assert cnt[b, hh] == len(tp_g["idx"])
            np.testing.assert_array_equal(idx[b, hh, :cnt[b, hh]], tp_g["idx"])
            d_ref, top_ref = chunk_dists(s_g, wl.D)
            np.testing.assert_array_equal(fd[j], d_ref[:L])
            np.testing.assert_array_equal(ft[j], top_ref)
            assert rel_err(o[b, hh], oracle.attend(s_g, codes, sz, wl.D, wl.Gv, tp_g["idx"])) <= 2e-3
            # end to end, from the oracle's own encoding
            assert rel_err(o[b, hh], r["out"]) <= 2e-3
            assert rel_err(of[b, hh], r["out_full"]) <= 2e-3
        _say(f"[full] unit {(b, h)} ok: cache identical={same}, kept {cnt[b, h * G:(h + 1) * G].tolist()}")

    # the step as the benchmark times it: tokens 0 .. L-2 appended, then one decode call that
    # appends token L-1 itself (its encoding inside the query-preparation launch)
    del cache, dbg
    cache2 = kvc.KVCache(npages, Hkv, R16, rot_kind=kind, page_size=wl.P, value_group=wl.Gv, device=dev)
    kvc.append(cache2, K[:, :L - 1].contiguous(), V[:, :L - 1].contiguous(), torch.zeros(B, dtype=torch.int32, device=dev),
               pt)
    out2 = kvc.decode_attend(cache2, q, seq, pt, top_p=wl.top_p, max_seq_len=L,
                             append=(K[:, L - 1:].contiguous(), V[:, L - 1:].contiguous(),
                                     torch.full((B,), L - 1, dtype=torch.int32, device=dev)))
    torch.cuda.synchronize()
    o2 = out2.cpu().numpy()
    kb2 = cache2.key_bits.cpu().numpy().view(np.uint32)
    for (b, h), (bits, nc, codes, sz, res) in zip(SAMPLED_UNITS, refs):
        pg, sl = pt_np[b, (L - 1) // wl.P], (L - 1) % wl.P
        np.testing.assert_array_equal(kb2[pg, h, sl], bits[L - 1])
        for j, hh in enumerate(range(h * G, (h + 1) * G)):
            assert rel_err(o2[b, hh], res[j]["out"]) <= 2e-3
    _say("[full] the benchmark's step (append inside the decode) ok")


def test_gqa_128k_topp_ragged_full_size():
    """The 128k GQA Top-p workload's shape (batch 4, 32 query / 8 KV heads, Top-p 0.9) with
    ragged lengths 131072, 130772, 70001 and 513, decoded as the benchmark runs it (no score
    output): enough 512-token chunks that a score wave covers two consecutive chunks, here
    with a sequence ending inside the first chunk of a pair and one inside the second.  The
    score pass's distances and chunk top bins, the Top-p counts, sets and outputs of sampled
    (sequence, KV head) units against the oracle run on the records the library wrote."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc

    wl = W.CONFIGS[2]
    dev = torch.device("cuda")
    B, Hq, Hkv, G = wl.B, wl.Hq, wl.Hkv, wl.Hq // wl.Hkv
    lens = np.array([131072, 131072 - 300, 70001, 513], np.int32)
    Lm = int(lens.max())
    _say(f"[full] {wl.name} ragged {lens.tolist()}: drawing inputs")
    K, V, q = W.draw_device(wl, dev, L=Lm)
    pt_np, npages = W.page_layout(wl, lens)
    kind, R16 = W.draw_rotation(wl)
    cache = kvc.KVCache(npages, Hkv, R16, rot_kind=kind, page_size=wl.P, value_group=wl.Gv, device=dev)
    pt = torch.from_numpy(pt_np).to(dev)
    for b in range(B):
        n = int(lens[b])
        kvc.append(cache, K[b:b + 1, :n].contiguous(), V[b:b + 1, :n].contiguous(),
                   torch.zeros(1, dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
    dbg = kvc.DecodeDebug.allocate(B, Hq, Lm, True, dev, scores=False, dist=True)
    out = kvc.decode_attend(cache, q, torch.from_numpy(lens).to(dev), pt, top_p=wl.top_p, max_seq_len=Lm,
                            debug=dbg)
    torch.cuda.synchronize()
    _say("[full] library decode done")
    assert torch.isfinite(out).all()
    orot = oracle.Rotation(oracle.ROT_DENSE, wl.D, R16=R16)
    kb = cache.key_bits.cpu().numpy().view(np.uint32)
    kn = cache.key_nc.cpu().numpy().view(np.uint32)
    vc = cache.val_codes.cpu().numpy()
    vs = cache.val_sz.cpu().numpy().view(np.uint32)
    o = out.cpu().numpy()
    qn = q.cpu().numpy()
    cnt = dbg.sel_count.cpu().numpy()
    for b, h in [(1, 2), (2, 5), (3, 7)]:
        n = int(lens[b])
        t = np.arange(n)
        pg, sl = pt_np[b, t // wl.P], t % wl.P
        ncw = kn[pg, h, sl]
        nc_g = np.stack([(ncw & 0xFFFF).astype(np.uint16), (ncw >> 16).astype(np.uint16)], axis=-1)
        codes = vc[pg, h, sl]
        szw = vs[pg, h, sl]
        sz = np.stack([(szw & 0xFFFF).astype(np.uint16), (szw >> 16).astype(np.uint16)], axis=-1)
        for hh in range(h * G, (h + 1) * G):
            qe = oracle.query_encode(orot, qn[b, hh][None, :])
            _, _, s_g = oracle.scores(kb[pg, h, sl], nc_g, qe["u"][0], qe["c0"][0], qe["c1"][0], wl.D)
            tp = oracle.topp(s_g, wl.top_p, wl.D)
            check_bins(dbg, b, hh, s_g, wl.D, Lm)
            assert cnt[b, hh] == len(tp["idx"]), (b, hh)
            np.testing.assert_array_equal(dbg.sel_idx[b, hh, :cnt[b, hh]].cpu().numpy(), tp["idx"])
            assert rel_err(o[b, hh], oracle.attend(s_g, codes, sz, wl.D, wl.Gv, tp["idx"])) <= 2e-3
        _say(f"[full] unit {(b, h)} over {n} tokens ok, kept {cnt[b, h * G:(h + 1) * G].tolist()}")


def test_7b_layer_full_size():
    """The 7B-shaped layer at its own shape: 32 heads x 8192 tokens, fp16 K/V with 4 outlier
    channels per head scaled by 8, dense rotation, full softmax.  Every head: the cache bytes
    against the oracle's encoding, the scores against the oracle on the library's records, and
    the outputs against the oracle; then the same cache under Top-p 0.9 (sets and the score
    pass's bins bit-exact)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc

    wl = W.CONFIGS[1]
    c = Case(wl)
    _say(f"[full] {wl.name}: oracle encode of {c.L} x {wl.Hkv} token-heads")
    c.ocache = c.oracle_cache()
    g = gpu_append(c)
    gb = download(g)
    stats = compare_caches(gb, c.ocache, c)
    _say(f"[full] cache ok {stats}")
    dev = torch.device("cuda")
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    og = oracle_cache_of(gb, c)
    for top_p in (1.0, 0.9):
        dbg = kvc.DecodeDebug.allocate(wl.B, wl.Hq, c.L, top_p < 1.0, dev, scores=top_p >= 1.0, dist=True)
        out = kvc.decode_attend(g, q, lens, pt, top_p=top_p, max_seq_len=c.L, debug=dbg).cpu().numpy()
        ref = c.oracle_decode(c.ocache, top_p)
        ref_g = c.oracle_decode(og, top_p)
        worst = 0.0
        for (b, h), r in ref_g.items():
            if top_p >= 1.0:
                np.testing.assert_array_equal(dbg.iscores[b, h].cpu().numpy(), r["A"])
                np.testing.assert_array_equal(dbg.scores[b, h].cpu().numpy().view(np.uint32), r["score"].view(np.uint32))
            else:
                cnt = int(dbg.sel_count[b, h])
                assert cnt == len(r["idx"]), (h, cnt, len(r["idx"]))
                np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
                check_bins(dbg, b, h, r["score"], wl.D, c.L)
            e = max(float(rel_err(out[b, h], r["out"])), float(rel_err(out[b, h], ref[(b, h)]["out"])))
            worst = max(worst, e)
            assert e <= 2e-3, (h, e)
        _say(f"[full] top_p={top_p}: every head ok, worst rel err {worst:.2e}")


def _check_unit_cache(kb, kn, vc, vs, pg, sl, h, bits, nc, codes, sz):
    """Cache bytes of one unit: sign words and norms exact, correction within one binary16
    ulp (its binary64 sum runs in another order), value codes and scale/zero exact.
    Returns whether the corrections are identical too."""
    np.testing.assert_array_equal(kb[pg, h, sl], bits)
    np.testing.assert_array_equal(kn[pg, h, sl] & 0xFFFF, nc[:, 0])
    assert np.all(np.abs((kn[pg, h, sl] >> 16).astype(np.int64) - nc[:, 1].astype(np.int64)) <= 1)
    np.testing.assert_array_equal(vc[pg, h, sl], codes)
    np.testing.assert_array_equal(vs[pg, h, sl], sz[..., 0].astype(np.uint32) | (sz[..., 1].astype(np.uint32) << 16))
    return bool(np.array_equal(kn[pg, h, sl] >> 16, nc[:, 1]))


def _oracle_encode(orot, k, v, D, Gv, threads=16):
    """The oracle's key and value encode of n tokens, split over host threads."""
    n = k.shape[0]
    cuts = np.linspace(0, n, threads + 1).astype(int)

    def part(i):
        a, b = cuts[i], cuts[i + 1]
        bits, nc = oracle.key_encode(orot, k[a:b])
        codes, sz = oracle.value_encode(v[a:b], D, Gv)
        return bits, nc, codes, sz

    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(part, range(threads)))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def test_batched_paged_full_size():
    """32 sequences x 32 heads, lengths uniform in [1024, 32768], shuffled 256-token pages,
    value group 64, full softmax: sampled (sequence, head) units against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc

    wl = W.CONFIGS[3]
    dev = torch.device("cuda")
    lens = W.draw_seq_lens(wl)
    Lm = int(lens.max())
    _say(f"[full] {wl.name}: drawing inputs, lengths {lens.min()}..{Lm}")
    K, V, q = W.draw_device(wl, dev, L=Lm)
    pt_np, npages = W.page_layout(wl, lens)
    kind, R16 = W.draw_rotation(wl)
    cache = kvc.KVCache(npages, wl.Hkv, R16, rot_kind=kind, page_size=wl.P, value_group=wl.Gv, device=dev)
    pt = torch.from_numpy(pt_np).to(dev)
    seq = torch.from_numpy(lens).to(dev)
    for b in range(wl.B):
        n = int(lens[b])
        kvc.append(cache, K[b:b + 1, :n].contiguous(), V[b:b + 1, :n].contiguous(),
                   torch.zeros(1, dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
    out = kvc.decode_attend(cache, q, seq, pt, top_p=1.0, max_seq_len=Lm)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    _say("[full] library decode done")
    orot = oracle.Rotation(oracle.ROT_DENSE, wl.D, R16=R16)
    kb = cache.key_bits.cpu().numpy().view(np.uint32)
    kn = cache.key_nc.cpu().numpy().view(np.uint32)
    vc = cache.val_codes.cpu().numpy()
    vs = cache.val_sz.cpu().numpy().view(np.uint32)
    o = out.cpu().numpy()
    qn = q.cpu().numpy()
    for b, h in [(int(np.argmax(lens)), 0), (int(np.argmin(lens)), 31), (7, 13)]:
        n = int(lens[b])
        k = K[b, :n, h].float().cpu().numpy()
        v = V[b, :n, h].float().cpu().numpy()
        bits, nc, codes, sz = _oracle_encode(orot, k, v, wl.D, wl.Gv)
        t = np.arange(n)
        pg, sl = pt_np[b, t // wl.P], t % wl.P
        _check_unit_cache(kb, kn, vc, vs, pg, sl, h, bits, nc, codes, sz)
        qe = oracle.query_encode(orot, qn[b, h][None, :])
        _, _, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], wl.D)
        ref = oracle.attend(s, codes, sz, wl.D, wl.Gv)
        assert rel_err(o[b, h], ref) <= 2e-3
        _say(f"[full] unit {(b, h)} ok over {n} tokens")


def test_append32k_and_decode1m_full_size():
    """The prefill append of 32768 tokens x 32 KV heads (randomized Hadamard rotation), then
    a decode over one 1,048,576-token sequence with 32 query / 8 KV heads and Top-p 0.95, its
    cache built by 32 appends of 32768 tokens: sampled heads against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc

    wl = W.CONFIGS[4]
    dev = torch.device("cuda")
    D, P, Gv = wl.D, wl.P, wl.Gv
    kind, signs = W.draw_rotation(wl)
    orot = oracle.Rotation(oracle.ROT_HADAMARD, D, signs=signs)

    # ---- prefill append, one call
    n_new, Ha = wl.append_tokens, wl.append_heads
    Ka, Va, _ = W.draw_device(wl, dev, L=n_new, Hkv=Ha)
    pta_np, npa = W.page_layout(wl.scaled(Hkv=Ha), np.array([n_new], np.int32))
    ca = kvc.KVCache(npa, Ha, signs, rot_kind=kind, page_size=P, value_group=Gv, device=dev)
    kvc.append(ca, Ka, Va, torch.zeros(1, dtype=torch.int32, device=dev), torch.from_numpy(pta_np).to(dev))
    torch.cuda.synchronize()
    kb = ca.key_bits.cpu().numpy().view(np.uint32)
    kn = ca.key_nc.cpu().numpy().view(np.uint32)
    vc = ca.val_codes.cpu().numpy()
    vs = ca.val_sz.cpu().numpy().view(np.uint32)
    t = np.arange(n_new)
    pg, sl = pta_np[0, t // P], t % P
    for h in (0, 31):
        enc = _oracle_encode(orot, Ka[0, :, h].float().cpu().numpy(), Va[0, :, h].float().cpu().numpy(), D, Gv)
        _check_unit_cache(kb, kn, vc, vs, pg, sl, h, *enc)
    _say(f"[full] append of {n_new} x {Ha} token-heads ok on sampled heads")
    del Ka, Va, ca, kb, kn, vc, vs

    # ---- 1M-token decode over 8 KV heads
    L, B, Hq, Hkv, G = wl.L, wl.B, wl.Hq, wl.Hkv, wl.Hq // wl.Hkv
    K, V, q = W.draw_device(wl, dev)
    lens = np.full(B, L, np.int32)
    pt_np, npages = W.page_layout(wl, lens)
    cache = kvc.KVCache(npages, Hkv, signs, rot_kind=kind, page_size=P, value_group=Gv, device=dev)
    pt = torch.from_numpy(pt_np).to(dev)
    for i in range(L // n_new):
        a = i * n_new
        kvc.append(cache, K[:, a:a + n_new].contiguous(), V[:, a:a + n_new].contiguous(),
                   torch.full((B,), a, dtype=torch.int32, device=dev), pt)
    seq = torch.from_numpy(lens).to(dev)
    dbg = kvc.DecodeDebug.allocate(B, Hq, L, True, dev, scores=False, dist=True)
    out = kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=L, debug=dbg)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    _say("[full] 1M-token decode done")
    cnt = dbg.sel_count.cpu().numpy()
    assert np.all(cnt >= 1) and np.all(cnt <= L)
    h = 5
    k = K[0, :, h].float().cpu().numpy()
    v = V[0, :, h].float().cpu().numpy()
    del K, V
    bits, nc, codes, sz = _oracle_encode(orot, k, v, D, Gv)
    kb = cache.key_bits[:, h].cpu().numpy().view(np.uint32)
    kn = cache.key_nc[:, h].cpu().numpy().view(np.uint32)
    t = np.arange(L)
    pg, sl = pt_np[0, t // P], t % P
    np.testing.assert_array_equal(kb[pg, sl], bits)
    np.testing.assert_array_equal(kn[pg, sl] & 0xFFFF, nc[:, 0])
    assert np.all(np.abs((kn[pg, sl] >> 16).astype(np.int64) - nc[:, 1].astype(np.int64)) <= 1)
    ncw = kn[pg, sl]
    nc_g = np.stack([(ncw & 0xFFFF).astype(np.uint16), (ncw >> 16).astype(np.uint16)], axis=-1)
    qn = q.cpu().numpy()
    o = out.cpu().numpy()
    for hh in range(h * G, (h + 1) * G):
        qe = oracle.query_encode(orot, qn[0, hh][None, :])
        # Top-p sets and the score pass's bins from the oracle on the library's records
        _, _, s_g = oracle.scores(kb[pg, sl], nc_g, qe["u"][0], qe["c0"][0], qe["c1"][0], D)
        tp_g = oracle.topp(s_g, wl.top_p, D)
        assert cnt[0, hh] == len(tp_g["idx"])
        np.testing.assert_array_equal(dbg.sel_idx[0, hh, :cnt[0, hh]].cpu().numpy(), tp_g["idx"])
        d_ref, top_ref = chunk_dists(s_g, D)
        np.testing.assert_array_equal(dbg.bin_dist[0, hh].cpu().numpy().view(np.uint16), d_ref[:L])
        np.testing.assert_array_equal(dbg.chunk_top[0, hh].cpu().numpy(), top_ref)
        # end to end from the oracle's own encoding
        _, _, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], D)
        tp = oracle.topp(s, wl.top_p, D)
        assert rel_err(o[0, hh], oracle.attend(s, codes, sz, D, Gv, tp["idx"])) <= 2e-3
        _say(f"[full] head {hh}: kept {cnt[0, hh]} of {L}")


def test_gqa_128k_exact_keys_full_size():
    """The 128k-context GQA Top-p workload with binary16 keys kept next to the compressed
    cache: the proxy scores select, the selected tokens are attended with exact scores.
    Sampled units: the binary16 keys and the outputs against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc

    wl = W.CONFIGS[2]
    dev = torch.device("cuda")
    B, Hq, Hkv, L, G = wl.B, wl.Hq, wl.Hkv, wl.L, wl.Hq // wl.Hkv
    _say(f"[full] {wl.name} with binary16 keys")
    K, V, q = W.draw_device(wl, dev)
    lens = np.full(B, L, np.int32)
    pt_np, npages = W.page_layout(wl, lens)
    kind, R16 = W.draw_rotation(wl)
    cache = kvc.KVCache(npages, Hkv, R16, rot_kind=kind, page_size=wl.P, value_group=wl.Gv, device=dev,
                        exact_keys=True)
    pt = torch.from_numpy(pt_np).to(dev)
    seq = torch.from_numpy(lens).to(dev)
    kvc.append(cache, K, V, torch.zeros(B, dtype=torch.int32, device=dev), pt)
    dbg = kvc.DecodeDebug.allocate(B, Hq, L, True, dev, scores=False)
    out = kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=L, debug=dbg)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    _say("[full] library decode done")
    cnt = dbg.sel_count.cpu().numpy()
    o = out.cpu().numpy()
    qn = q.cpu().numpy()
    vc = cache.val_codes.cpu().numpy()
    vs = cache.val_sz.cpu().numpy().view(np.uint32)
    kb = cache.key_bits.cpu().numpy().view(np.uint32)
    kn = cache.key_nc.cpu().numpy().view(np.uint32)
    orot = oracle.Rotation(oracle.ROT_DENSE, wl.D, R16=R16)
    for b, h in [(1, 2), (2, 5)]:
        t = np.arange(L)
        pg, sl = pt_np[b, t // wl.P], t % wl.P
        k16 = cache.keys_f16[:, h].cpu().numpy()[pg, sl]
        np.testing.assert_array_equal(k16.view(np.uint16), K[b, :, h].cpu().numpy().view(np.uint16))
        codes = vc[pg, h, sl]
        szw = vs[pg, h, sl]
        sz = np.stack([(szw & 0xFFFF).astype(np.uint16), (szw >> 16).astype(np.uint16)], axis=-1)
        ncw = kn[pg, h, sl]
        nc_g = np.stack([(ncw & 0xFFFF).astype(np.uint16), (ncw >> 16).astype(np.uint16)], axis=-1)
        for hh in range(h * G, (h + 1) * G):
            # the set the oracle's Top-p chooses on the library's records, not the library's own
            qe = oracle.query_encode(orot, qn[b, hh][None, :])
            _, _, s_g = oracle.scores(kb[pg, h, sl], nc_g, qe["u"][0], qe["c0"][0], qe["c1"][0], wl.D)
            idx = oracle.topp(s_g, wl.top_p, wl.D)["idx"]
            assert cnt[b, hh] == len(idx)
            np.testing.assert_array_equal(dbg.sel_idx[b, hh, :cnt[b, hh]].cpu().numpy(), idx)
            ref = oracle.attend_exact(qn[b, hh], k16, codes, sz, wl.D, wl.Gv, idx)
            assert rel_err(o[b, hh], ref) <= 2e-3
        _say(f"[full] unit {(b, h)} ok, kept {cnt[b, h * G:(h + 1) * G].tolist()}")
