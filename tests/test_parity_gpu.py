"""GPU parity of the library (through its C ABI) against the oracle, on seeded synthetic
workloads at sizes the oracle finishes in seconds (several chunks and pages, ragged tails,
empty and one-token sequences, GQA groups 1/2/4/8, both rotations, value groups 32/64).

Bars: bit-exact for every byte of the cache, the int4 query codes and parameters, the
integer scores, the binary32 proxy scores, and the Top-p counts, thresholds and index sets;
attention outputs within 2e-3 of the oracle's binary64 output, as
max_j |out - ref| / max_j |ref| per (sequence, query head).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from tests.kvc_testlib import (Case, check_bins, compare_caches, download, gpu_append, oracle_cache_of, rel_err,
                               upload)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def _cases():
    return {
        "c1-full-fp32-dense": dict(wl=W.CONFIGS[0]),
        "c2-outliers-ragged": dict(wl=W.CONFIGS[1].scaled(Hq=4, Hkv=4, P=64), L=1000),
        "c3-gqa4-spikes-topp": dict(wl=W.CONFIGS[2].scaled(B=2, Hq=8, Hkv=2, P=128), L=3000),
        "c4-paged-g64-ragged": dict(wl=W.CONFIGS[3].scaled(B=5, Hq=4, Hkv=4), L=2500,
                                    seq_lens=[2500, 0, 1, 777, 2049]),
        "c5-hadamard-topp": dict(wl=W.CONFIGS[4].scaled(Hq=8, Hkv=2), L=5000),
        "gqa2-pages16-p0.5": dict(wl=W.CONFIGS[2].scaled(B=1, Hq=4, Hkv=2, P=16, top_p=0.5), L=1500),
        "gqa8-topp": dict(wl=W.CONFIGS[2].scaled(B=1, Hq=16, Hkv=2), L=2000),
    }


CASES = _cases()
_built = {}


def _case(name):
    if name not in _built:
        spec = dict(CASES[name])
        wl = spec.pop("wl")
        c = Case(wl, **spec)
        c.ocache = c.oracle_cache()
        _built[name] = c
    return _built[name]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_kv_cache_compress_amd as kvc  # noqa: F401  (fails loudly if the library is missing)

    yield


@pytest.mark.parametrize("name", list(CASES))
def test_append_parity(name):
    c = _case(name)
    _say(f"[append] {name} B={c.wl.B} L={c.L} Hkv={c.wl.Hkv} rot={c.rot_kind} dtype={c.wl.kv_dtype}")
    g = gpu_append(c)
    stats = compare_caches(download(g), c.ocache, c)
    _say(f"[append] {name} ok {stats}")


def test_dense_append_certified_signs():
    """The dense rotation on the matrix cores (more than 8192 binary16 token-heads) with keys
    built so that many rotated coordinates sit at or near zero, where the binary32 sums cannot
    certify a sign and the binary64 sum decides: zero keys (every coordinate uncertain, each
    sign +1), one-hot keys (k' is a column of R), the columns of R themselves (k' = R R^T e_i,
    which is e_i up to the binary16 rounding of R) and their negatives, beside random keys.
    Every record against the oracle's encoding (sign bits exact outside the 2^-40 band)."""
    wl = W.CONFIGS[2].scaled(B=1, Hq=8, Hkv=8, P=256)
    c = Case(wl, L=2048)  # 16384 token-heads: the matrix-core append
    assert c.rot_kind == "dense"
    R = c.rot_raw.astype(np.float16)
    K = c.K
    for t in range(c.L):
        for h in range(wl.Hkv):
            kind, i = (t + h) % 5, (7 * t + 3 * h) % wl.D
            if kind == 0:
                K[0, t, h] = 0.0
            elif kind == 1:
                K[0, t, h] = 0.0
                K[0, t, h, i] = np.float16(1.5 + (t % 7))
            elif kind == 2:
                K[0, t, h] = R[:, i]
            elif kind == 3:
                K[0, t, h] = -R[:, i]
    c.ocache = c.oracle_cache()
    g = gpu_append(c)
    d = download(g)
    stats = compare_caches(d, c.ocache, c)
    # zero keys exactly: every sign +1 (a zero counts as positive), norm 0, correction 1
    for t in range(c.L):
        for h in range(wl.Hkv):
            if (t + h) % 5 == 0:
                pg, sl = c.pt[0, t // wl.P], t % wl.P
                assert np.all(d["key_bits"][pg, h, sl] == 0xFFFFFFFF), (t, h)
                assert int(d["key_nc"][pg, h, sl]) == 0x3C000000, (t, h, hex(int(d["key_nc"][pg, h, sl])))
    _say(f"[append] certified signs ok {stats}")


def _decode_with_debug(c, cache, top_p, scores=True, proxy=False, dist=True):
    """Decode with debug outputs; scores=False runs the kernels of a decode without debug
    output (the per-token scores are not written) and still returns the Top-p sets and what
    the score pass wrote (bin distances, chunk top bins)."""
    from bit_kv_cache_compress_amd import DecodeDebug, decode_attend

    dev = torch.device("cuda")
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    dbg = DecodeDebug.allocate(c.wl.B, c.wl.Hq, c.max_len, top_p < 1.0, dev, scores=scores, dist=dist)
    out = decode_attend(cache, q, lens, pt, top_p=top_p, max_seq_len=c.max_len, debug=dbg, proxy=proxy)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dbg


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["config", "full"])
def test_decode_stagewise(name, mode):
    """The library's decode on the oracle's cache bytes, stage by stage."""
    c = _case(name)
    top_p = c.wl.top_p if mode == "config" else 1.0
    _say(f"[decode] {name} top_p={top_p}")
    g = upload(c.ocache, c)
    out, dbg = _decode_with_debug(c, g, top_p)
    ref = c.oracle_decode(c.ocache, top_p)
    qc = dbg.q_codes.cpu().numpy()
    qp = dbg.q_params.cpu().numpy()
    qs = dbg.q_sumu.cpu().numpy()
    A = dbg.iscores.cpu().numpy()
    S = dbg.scores.cpu().numpy()
    worst = 0.0
    for (b, h), r in ref.items():
        np.testing.assert_array_equal(qc[b, h], r["u"])
        np.testing.assert_array_equal(qp[b, h], np.array([r["vl"], r["delta"], r["c0"], r["c1"]], np.float32))
        assert qs[b, h] == r["sumu"]
        n = int(c.lens[b])
        np.testing.assert_array_equal(A[b, h, :n], r["A"])
        np.testing.assert_array_equal(S[b, h, :n].view(np.uint32), r["score"].view(np.uint32))
        if top_p < 1.0 and n > 0:
            cnt = int(dbg.sel_count[b, h])
            assert cnt == len(r["idx"]), (b, h, cnt, len(r["idx"]))
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            bins = dbg.sel_bins[b, h].cpu().numpy()
            assert (int(bins[0]), int(bins[1])) == (r["emax"], r["bstar"])
            check_bins(dbg, b, h, r["score"], c.wl.D, c.max_len)
        e = float(rel_err(out[b, h], r["out"])) if n else float(np.abs(out[b, h]).max())
        if n == 0:
            assert e == 0.0
        worst = max(worst, e)
        assert e <= TOL, (b, h, e)
    _say(f"[decode] {name} top_p={top_p} ok, worst rel err {worst:.2e}")


@pytest.mark.parametrize("name", list(CASES))
def test_end_to_end(name):
    """Library append + decode from raw K/V against oracle append + decode."""
    c = _case(name)
    _say(f"[e2e] {name}")
    g = gpu_append(c)
    gb = download(g)
    same = all(np.array_equal(v, getattr(c.ocache, k)) for k, v in gb.items())
    out, dbg = _decode_with_debug(c, g, c.wl.top_p, scores=False)
    ref = c.oracle_decode(c.ocache, c.wl.top_p)
    worst = max(float(rel_err(out[b, h], r["out"])) if int(c.lens[b]) else 0.0 for (b, h), r in ref.items())
    assert worst <= TOL
    # the oracle's query encode, scores, Top-p and attention on the bytes the library wrote:
    # every set, bin and threshold bit-exact whatever the encoders' rounding did
    ref_g = c.oracle_decode(oracle_cache_of(gb, c), c.wl.top_p)
    for (b, h), r in ref_g.items():
        n = int(c.lens[b])
        if n:
            assert rel_err(out[b, h], r["out"]) <= TOL
        if c.wl.top_p < 1.0 and n:
            cnt = int(dbg.sel_count[b, h])
            assert cnt == len(r["idx"]), (b, h, cnt, len(r["idx"]))
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            bins = dbg.sel_bins[b, h].cpu().numpy()
            assert (int(bins[0]), int(bins[1])) == (r["emax"], r["bstar"])
            check_bins(dbg, b, h, r["score"], c.wl.D, c.max_len)
    _say(f"[e2e] {name} ok, caches identical={same}, worst rel err {worst:.2e}")


@pytest.mark.parametrize("name", [n for n in CASES if CASES[n]["wl"].top_p < 1.0])
def test_score_kernels_agree(name):
    """The Top-p score pass of a decode without score output (the matrix-core kernel for
    GQA groups of 4 or more) against the debug score pass (dot8): identical top bins,
    thresholds, Top-p sets and bit-identical outputs on the oracle's cache."""
    c = _case(name)
    _say(f"[kernels] {name}")
    g = upload(c.ocache, c)
    o_dbg, d_dbg = _decode_with_debug(c, g, c.wl.top_p)
    o_fast, d_fast = _decode_with_debug(c, g, c.wl.top_p, scores=False)
    np.testing.assert_array_equal(d_fast.sel_count.cpu().numpy(), d_dbg.sel_count.cpu().numpy())
    np.testing.assert_array_equal(d_fast.sel_bins.cpu().numpy(), d_dbg.sel_bins.cpu().numpy())
    np.testing.assert_array_equal(d_fast.sel_idx.cpu().numpy(), d_dbg.sel_idx.cpu().numpy())
    assert np.array_equal(o_fast.view(np.uint32), o_dbg.view(np.uint32))
    # the fast kernels' own output, per token: bins of every query head against the oracle's
    ref = c.oracle_decode(c.ocache, c.wl.top_p)
    for (b, h), r in ref.items():
        if int(c.lens[b]):
            check_bins(d_fast, b, h, r["score"], c.wl.D, c.max_len)
    _say(f"[kernels] {name} ok")


@pytest.mark.parametrize("name", [n for n in CASES if CASES[n]["wl"].top_p < 1.0])
def test_exact_keys(name):
    """Binary16 keys next to the compressed cache: the appended bytes equal the oracle's
    (nearest-even rounding of the input); a Top-p decode keeps the proxy sets and attends them
    with the exact scores <q, k>; proxy=True gives the proxy-score output."""
    c = _case(name)
    _say(f"[exact] {name}")
    oc = c.oracle_cache(exact_keys=True)
    g = gpu_append(c, exact_keys=True)
    np.testing.assert_array_equal(g.keys_f16.cpu().numpy().view(np.uint16), oc.key_f16.view(np.uint16))
    g = upload(oc, c)
    ref = c.oracle_decode(oc, c.wl.top_p)
    out, dbg = _decode_with_debug(c, g, c.wl.top_p, scores=False)
    out_p, _ = _decode_with_debug(c, g, c.wl.top_p, scores=False, proxy=True)
    worst = 0.0
    for (b, h), r in ref.items():
        if int(c.lens[b]) == 0:
            assert np.abs(out[b, h]).max() == 0.0
            continue
        cnt = int(dbg.sel_count[b, h])
        np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
        e = float(rel_err(out[b, h], r["out"]))
        worst = max(worst, e)
        assert e <= TOL, (b, h, e)
        assert rel_err(out_p[b, h], r["out_proxy"]) <= TOL
    _say(f"[exact] {name} ok, worst rel err {worst:.2e}")


@pytest.mark.parametrize("name", ["c2-outliers-ragged", "c3-gqa4-spikes-topp", "c4-paged-g64-ragged",
                                  "c5-hadamard-topp"])
def test_tail(name):
    """The compressed cache plus a binary16 tail of uncompressed recent tokens (lazy updates):
    tail lengths 0, 1, 100 and a whole 256-token page, one softmax over both, at the case's
    Top-p and with full softmax, against the oracle."""
    import oracle
    from bit_kv_cache_compress_amd import Tail, decode_attend

    c = _case(name)
    dev = torch.device("cuda")
    B, Hkv, D, cap = c.wl.B, c.wl.Hkv, c.wl.D, 256
    ntail = np.minimum(np.array([[0, 1, 100, 256][b % 4] for b in range(B)], np.int32), c.lens)
    lc = (c.lens - ntail).astype(np.int32)
    tk = np.zeros((B, cap, Hkv, D), np.float16)
    tv = np.zeros_like(tk)
    for b in range(B):
        tk[b, :ntail[b]] = c.K[b, lc[b]:lc[b] + ntail[b]].astype(np.float16)
        tv[b, :ntail[b]] = c.V[b, lc[b]:lc[b] + ntail[b]].astype(np.float16)
    tail = Tail(B, cap, Hkv, dev)
    tail.k.copy_(torch.from_numpy(tk))
    tail.v.copy_(torch.from_numpy(tv))
    tail.len.copy_(torch.from_numpy(ntail))
    g = upload(c.ocache, c)
    q = torch.from_numpy(c.q).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    lcd = torch.from_numpy(lc).to(dev)
    for top_p in sorted({c.wl.top_p, 1.0}):
        _say(f"[tail] {name} top_p={top_p} tails {ntail.tolist()}")
        out = decode_attend(g, q, lcd, pt, top_p=top_p, max_seq_len=c.max_len, tail=tail)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref = oracle.decode(c.ocache, c.orot, c.q, lc, c.pt, top_p, tail=(tk, tv, ntail))
        worst = 0.0
        for (b, h), r in ref.items():
            if lc[b] + ntail[b] == 0:
                assert np.abs(out[b, h]).max() == 0.0
                continue
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (top_p, b, h, e)
        _say(f"[tail] {name} top_p={top_p} ok, worst rel err {worst:.2e}")


def test_tail_append_and_retire():
    """Tail maintenance: appended tokens are the binary16 roundings of the input (float32 and
    float16), past-capacity tokens are dropped, and retiring moves the rest to the front
    (including moves whose source and destination ranges overlap) and advances seq_lens."""
    from bit_kv_cache_compress_amd import Tail

    dev = torch.device("cuda")
    rng = np.random.default_rng(7)
    B, Hkv, D, cap = 3, 2, 128, 40
    tail = Tail(B, cap, Hkv, dev)
    want_k = np.zeros((B, cap, Hkv, D), np.float16)
    want_v = np.zeros_like(want_k)
    lens = np.zeros(B, np.int64)
    for n, dt in [(5, np.float32), (1, np.float16), (30, np.float32), (7, np.float16)]:
        k = (3 * rng.standard_normal((B, n, Hkv, D))).astype(dt)
        v = rng.standard_normal((B, n, Hkv, D)).astype(dt)
        tail.append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev))
        for b in range(B):
            m = min(n, cap - lens[b])
            want_k[b, lens[b]:lens[b] + m] = k[b, :m].astype(np.float16)
            want_v[b, lens[b]:lens[b] + m] = v[b, :m].astype(np.float16)
            lens[b] += m
    torch.cuda.synchronize()
    assert tail.len.cpu().numpy().tolist() == lens.tolist() == [cap] * B
    np.testing.assert_array_equal(tail.k.cpu().numpy().view(np.uint16), want_k.view(np.uint16))
    np.testing.assert_array_equal(tail.v.cpu().numpy().view(np.uint16), want_v.view(np.uint16))
    seq = torch.tensor([100, 0, 7], dtype=torch.int32, device=dev)
    for n in (3, 16):  # 37 kept after 3 (overlapping move), then 21 after 16
        tail.retire(n, seq)
        torch.cuda.synchronize()
        want_k = np.concatenate([want_k[:, n:], np.zeros_like(want_k[:, :n])], axis=1)
        want_v = np.concatenate([want_v[:, n:], np.zeros_like(want_v[:, :n])], axis=1)
        lens -= n
        assert tail.len.cpu().numpy().tolist() == lens.tolist()
        got_k, got_v = tail.k.cpu().numpy(), tail.v.cpu().numpy()
        for b in range(B):
            np.testing.assert_array_equal(got_k[b, :lens[b]].view(np.uint16), want_k[b, :lens[b]].view(np.uint16))
            np.testing.assert_array_equal(got_v[b, :lens[b]].view(np.uint16), want_v[b, :lens[b]].view(np.uint16))
    assert seq.cpu().numpy().tolist() == [119, 19, 26]


def test_lazy_pipeline():
    """Lazy updates end to end: tokens go to the binary16 tail one step at a time, a whole page
    of the tail is compressed on a second stream while decodes go on, then retired; every
    step's output (cache plus tail) against the oracle holding the same state."""
    import oracle
    from bit_kv_cache_compress_amd import Tail, append, decode_attend

    c = _case("c3-gqa4-spikes-topp")  # binary16 inputs: the tail keeps them exactly
    dev = torch.device("cuda")
    B, Hkv, D, P = c.wl.B, c.wl.Hkv, c.wl.D, c.wl.P
    L0 = 2 * P + 5                     # compressed at the start
    steps = P + 9                      # one page fills and is compressed on the way
    assert L0 + steps <= c.L
    ocache = oracle.PagedCache(c.npages, Hkv, P, D, c.wl.Gv)
    oracle.append(ocache, c.orot, c.K[:, :L0], c.V[:, :L0], np.zeros(B, np.int32), c.pt)
    g = upload(ocache, c)
    tail = Tail(B, 2 * P, Hkv, dev)
    seq = torch.full((B,), L0, dtype=torch.int32, device=dev)
    pt = torch.from_numpy(c.pt).to(dev)
    q = torch.from_numpy(c.q).to(dev)
    side = torch.cuda.Stream()
    lc, nt, pending = L0, 0, None
    for s in range(steps):
        t = L0 + s
        tail.append(torch.from_numpy(np.ascontiguousarray(c.K[:, t:t + 1])).to(dev),
                    torch.from_numpy(np.ascontiguousarray(c.V[:, t:t + 1])).to(dev))
        nt += 1
        if nt == P + 1 and pending is None:
            # the tail's first page (positions lc .. lc+P-1) is compressed on the side stream
            ev = torch.cuda.Event()
            ev.record()
            side.wait_event(ev)
            with torch.cuda.stream(side):
                for b in range(B):
                    kb, vb = tail.page(b, 0, P)
                    append(g, kb, vb, torch.tensor([lc], dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
                done = torch.cuda.Event()
                done.record()
            pending = (done, s + 4)
        if pending is not None and s == pending[1]:
            torch.cuda.current_stream().wait_event(pending[0])
            tail.retire(P, seq)
            oracle.append(ocache, c.orot, c.K[:, lc:lc + P], c.V[:, lc:lc + P], np.full(B, lc, np.int32), c.pt)
            lc, nt, pending = lc + P, nt - P, None
        out = decode_attend(g, q, seq, pt, top_p=c.wl.top_p, max_seq_len=c.L, tail=tail)
        if s % 40 == 0 or s == steps - 1:
            torch.cuda.synchronize()
            tk = np.zeros((B, 2 * P, Hkv, D), np.float16)
            tv = np.zeros_like(tk)
            tk[:, :nt] = c.K[:, lc:lc + nt].astype(np.float16)
            tv[:, :nt] = c.V[:, lc:lc + nt].astype(np.float16)
            ref = oracle.decode(ocache, c.orot, c.q, np.full(B, lc, np.int32), c.pt, c.wl.top_p,
                                tail=(tk, tv, np.full(B, nt, np.int32)))
            o = out.cpu().numpy()
            for (b, h), r in ref.items():
                assert rel_err(o[b, h], r["out"]) <= TOL, (s, b, h)
            _say(f"[lazy] step {s}: {lc} compressed + {nt} tail tokens ok")
    assert lc == L0 + P and int(seq[0]) == lc


def test_topp_sweep():
    """Top-p from 0.3 to 0.999 on one cache (from a few dozen to almost every token of a
    1024-token attention chunk kept): sets and outputs against the oracle."""
    c = _case("c5-hadamard-topp")
    for top_p in (0.3, 0.45, 0.6, 0.8, 0.95, 0.999):
        _say(f"[sweep] top_p={top_p}")
        g = upload(c.ocache, c)
        out, dbg = _decode_with_debug(c, g, top_p, scores=False)
        ref = c.oracle_decode(c.ocache, top_p)
        for (b, h), r in ref.items():
            cnt = int(dbg.sel_count[b, h])
            assert cnt == len(r["idx"]), (top_p, b, h, cnt, len(r["idx"]))
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            assert rel_err(out[b, h], r["out"]) <= TOL, (top_p, b, h)
    _say("[sweep] ok")


def test_chunked_append_and_determinism():
    c = _case("c3-gqa4-spikes-topp")
    _say("[chunks] chunked append 1/7/300-token pieces and repeated decode")
    whole = download(gpu_append(c))
    for chunk in (1, 7, 300):
        part = download(gpu_append(c, chunk=chunk))
        for k in whole:
            np.testing.assert_array_equal(part[k], whole[k])
    g = upload(c.ocache, c)
    o1, _ = _decode_with_debug(c, g, c.wl.top_p)
    o2, _ = _decode_with_debug(c, g, c.wl.top_p)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    _say("[chunks] ok")


def test_topp_select_standalone():
    import oracle
    from bit_kv_cache_compress_amd import topp_select

    rng = np.random.default_rng(77)
    B, Hq, ld = 3, 5, 7000
    lens = np.array([7000, 1, 4321], np.int32)
    s = (rng.standard_normal((B, Hq, ld)) * np.sqrt(128)).astype(np.float32)
    s[0, 1, :] = 2.5                                  # all equal: everything kept
    s[2, 2, 1234] = 500.0                             # one dominant token
    s[0, 3, ::3] += 60.0                              # a third of the tokens boosted
    _say("[topp] standalone selection")
    for p in (0.05, 0.5, 0.9, 0.999):
        idx, cnt = topp_select(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), p)
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for b in range(B):
            for h in range(Hq):
                r = oracle.topp(s[b, h, :lens[b]], p, 128)
                assert cnt[b, h] == len(r["idx"]), (p, b, h)
                np.testing.assert_array_equal(idx[b, h, :cnt[b, h]], r["idx"])
                assert np.all(idx[b, h, cnt[b, h]:] == -1)
    _say("[topp] ok")


def _centers(c):
    """Per-KV-head key centers: the mean of the case's keys (binary32), as a caller would
    take it from the prefill."""
    m = np.zeros((c.wl.Hkv, c.wl.D), np.float64)
    n = 0
    for b in range(c.wl.B):
        L = int(c.lens[b])
        m += c.K[b, :L].astype(np.float64).sum(axis=0)
        n += L
    return (m / max(n, 1)).astype(np.float32)


def _tail_of(c, ntail, cap, dev):
    """A binary16 tail holding tokens lens-ntail .. lens-1 of each sequence (the compressed
    length becomes lens - ntail)."""
    from bit_kv_cache_compress_amd import Tail

    B, Hkv, D = c.wl.B, c.wl.Hkv, c.wl.D
    lc = (c.lens - ntail).astype(np.int32)
    tk = np.zeros((B, cap, Hkv, D), np.float16)
    tv = np.zeros_like(tk)
    for b in range(B):
        tk[b, :ntail[b]] = c.K[b, lc[b]:lc[b] + ntail[b]].astype(np.float16)
        tv[b, :ntail[b]] = c.V[b, lc[b]:lc[b] + ntail[b]].astype(np.float16)
    tail = Tail(B, cap, Hkv, dev)
    tail.k.copy_(torch.from_numpy(tk))
    tail.v.copy_(torch.from_numpy(tv))
    tail.len.copy_(torch.from_numpy(ntail.astype(np.int32)))
    return tail, (tk, tv, ntail), lc


@pytest.mark.parametrize("name", ["c1-full-fp32-dense", "c2-outliers-ragged", "c3-gqa4-spikes-topp",
                                  "c4-paged-g64-ragged", "c5-hadamard-topp"])
def test_key_centering(name):
    """Per-head key centering: the appended cache bytes bit-exact against the oracle's
    centered cache, the decode's codes, proxy scores and Top-p sets bit-exact, outputs
    within the bar, also with a binary16 tail (scores moved into the centered frame) and,
    under Top-p, with exact scores."""
    from bit_kv_cache_compress_amd import decode_attend

    c = _case(name)
    dev = torch.device("cuda")
    kc = _centers(c)
    _say(f"[center] {name} |c| max {np.abs(kc).max():.3f}")
    ocen = c.oracle_cache(key_center=kc)
    g = gpu_append(c, key_center=torch.from_numpy(kc))
    stats = compare_caches(download(g), ocen, c)
    _say(f"[center] {name} append ok {stats}")
    gu = upload(ocen, c)
    for top_p in sorted({c.wl.top_p, 1.0}):
        out, dbg = _decode_with_debug(c, gu, top_p)
        ref = oracle.decode(ocen, c.orot, c.q, c.lens, c.pt, top_p)
        S = dbg.scores.cpu().numpy()
        worst = 0.0
        for (b, h), r in ref.items():
            n = int(c.lens[b])
            np.testing.assert_array_equal(S[b, h, :n].view(np.uint32), r["score"].view(np.uint32))
            if top_p < 1.0 and n > 0:
                cnt = int(dbg.sel_count[b, h])
                np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            if n == 0:
                assert np.abs(out[b, h]).max() == 0.0
                continue
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (top_p, b, h, e)
        _say(f"[center] {name} top_p={top_p} ok, worst rel err {worst:.2e}")
    # with a tail, proxy and (under Top-p) exact scores
    ntail = np.minimum(np.array([[0, 1, 100, 256][b % 4] for b in range(c.wl.B)], np.int32), c.lens)
    tail, otail, lc = _tail_of(c, ntail, 256, dev)
    lcd = torch.from_numpy(lc).to(dev)
    q = torch.from_numpy(c.q).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    variants = [(False, top_p) for top_p in sorted({c.wl.top_p, 1.0})]
    if c.wl.top_p < 1.0:
        variants.append((True, c.wl.top_p))
    for exact, top_p in variants:
        oc = c.oracle_cache(exact_keys=True, key_center=kc) if exact else ocen
        gc = upload(oc, c) if exact else gu
        out = decode_attend(gc, q, lcd, pt, top_p=top_p, max_seq_len=c.max_len, tail=tail)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref = oracle.decode(oc, c.orot, c.q, lc, c.pt, top_p, tail=otail)
        worst = 0.0
        for (b, h), r in ref.items():
            if lc[b] + ntail[b] == 0:
                assert np.abs(out[b, h]).max() == 0.0
                continue
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (exact, top_p, b, h, e)
        _say(f"[center] {name} tail exact={exact} top_p={top_p} ok, worst rel err {worst:.2e}")


@pytest.mark.parametrize("name", ["c2-outliers-ragged", "c3-gqa4-spikes-topp", "c4-paged-g64-ragged",
                                  "c5-hadamard-topp", "gqa8-topp"])
def test_stochastic_query_rounding(name):
    """Seeded stochastic rounding of the int4 query (uniforms passed in): codes, parameters,
    scores and Top-p sets bit-exact against the oracle given the same uniforms, outputs
    within the bar; with a tail too."""
    from bit_kv_cache_compress_amd import DecodeDebug, decode_attend

    c = _case(name)
    dev = torch.device("cuda")
    rng = np.random.default_rng(1234)
    U = rng.random((c.wl.B, c.wl.Hq, c.wl.D), dtype=np.float32)
    Ud = torch.from_numpy(U).to(dev)
    g = upload(c.ocache, c)
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    for top_p in sorted({c.wl.top_p, 1.0}):
        _say(f"[dither] {name} top_p={top_p}")
        dbg = DecodeDebug.allocate(c.wl.B, c.wl.Hq, c.max_len, top_p < 1.0, dev)
        out = decode_attend(g, q, lens, pt, top_p=top_p, max_seq_len=c.max_len, debug=dbg, q_dither=Ud)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref = oracle.decode(c.ocache, c.orot, c.q, c.lens, c.pt, top_p, dither=U)
        plain = c.oracle_decode(c.ocache, top_p)
        qc = dbg.q_codes.cpu().numpy()
        qp = dbg.q_params.cpu().numpy()
        S = dbg.scores.cpu().numpy()
        worst, differ = 0.0, 0
        for (b, h), r in ref.items():
            np.testing.assert_array_equal(qc[b, h], r["u"])
            np.testing.assert_array_equal(qp[b, h], np.array([r["vl"], r["delta"], r["c0"], r["c1"]], np.float32))
            differ += int(np.any(r["u"] != plain[(b, h)]["u"]))
            n = int(c.lens[b])
            np.testing.assert_array_equal(S[b, h, :n].view(np.uint32), r["score"].view(np.uint32))
            if top_p < 1.0 and n > 0:
                cnt = int(dbg.sel_count[b, h])
                np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            if n == 0:
                assert np.abs(out[b, h]).max() == 0.0
                continue
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (top_p, b, h, e)
        assert differ > 0  # the dither changed the codes
        _say(f"[dither] {name} top_p={top_p} ok, worst rel err {worst:.2e}")
    ntail = np.minimum(np.array([[0, 1, 100, 256][b % 4] for b in range(c.wl.B)], np.int32), c.lens)
    tail, otail, lc = _tail_of(c, ntail, 256, dev)
    out = decode_attend(g, q, torch.from_numpy(lc).to(dev), pt, top_p=c.wl.top_p, max_seq_len=c.max_len,
                        tail=tail, q_dither=Ud)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = oracle.decode(c.ocache, c.orot, c.q, lc, c.pt, c.wl.top_p, tail=otail, dither=U)
    for (b, h), r in ref.items():
        if lc[b] + ntail[b] == 0:
            continue
        assert rel_err(out[b, h], r["out"]) <= TOL, (b, h)
    _say(f"[dither] {name} tail ok")


def _tier_case(c, lc, C, seed, sketch=None):
    """An oracle cache copy with, per (sequence, KV head), up to 5 of its compressed tokens moved
    into a high-precision tier of C entries (scattered slots), and the same state on the GPU."""
    import copy

    from bit_kv_cache_compress_amd import HPTier

    rng = np.random.default_rng(seed)
    B, Hkv, D = c.wl.B, c.wl.Hkv, c.wl.D
    oc = copy.deepcopy(c.ocache) if sketch is None else c.oracle_cache(sketch=sketch)
    hp = oracle.HPTier(B, Hkv, C, D)
    slots = [1, 3, 4, 6, 7]
    for b in range(B):
        for h in range(Hkv):
            n = min(5, int(lc[b]))
            for i, t in enumerate(sorted(rng.choice(int(lc[b]), n, replace=False).tolist()) if n else []):
                pg, sl = oc.locate(b, t, c.pt)
                f = slots[i]
                hp.saved[b, h, f] = oc.key_nc[pg, h, sl]
                oc.key_nc[pg, h, sl] = oracle.HPTier.MARKER
                hp.pos[b, h, f] = t
                hp.k16[b, h, f] = c.K[b, t, h].astype(np.float16)
                hp.v16[b, h, f] = c.V[b, t, h].astype(np.float16)
    dev = torch.device("cuda")
    g = upload(oc, c)
    hg = HPTier(B, C, Hkv, dev)
    hg.k.copy_(torch.from_numpy(hp.k16))
    hg.v.copy_(torch.from_numpy(hp.v16))
    hg.pos.copy_(torch.from_numpy(hp.pos.astype(np.int32)))
    hg.saved.copy_(torch.from_numpy(hp.saved.view(np.int32)))
    return oc, hp, g, hg


@pytest.mark.parametrize("name", ["c2-outliers-ragged", "c3-gqa4-spikes-topp", "c4-paged-g64-ragged",
                                  "c5-hadamard-topp"])
def test_hp_tier_decode(name):
    """Decode with the high-precision tier and a tail: outputs within the bar against the
    oracle, and the masses the decode adds to tail tokens and tier entries within 1e-3
    (relative) of the oracle's binary64 weights, summed over each KV head's query heads."""
    from bit_kv_cache_compress_amd import decode_attend

    c = _case(name)
    dev = torch.device("cuda")
    B, Hkv = c.wl.B, c.wl.Hkv
    ntail = np.minimum(np.array([[0, 1, 100, 256][b % 4] for b in range(B)], np.int32), c.lens)
    lc = (c.lens - ntail).astype(np.int32)
    oc, hp, g, hg = _tier_case(c, lc, 8, 31)
    tail, otail, _ = _tail_of(c, ntail, 256, dev)
    from bit_kv_cache_compress_amd import Tail
    tailm = Tail(B, 256, Hkv, dev, mass=True)
    tailm.k.copy_(tail.k)
    tailm.v.copy_(tail.v)
    tailm.len.copy_(tail.len)
    q = torch.from_numpy(c.q).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    lcd = torch.from_numpy(lc).to(dev)
    for top_p in sorted({c.wl.top_p, 1.0}):
        tailm.mass.zero_()
        hg.mass.zero_()
        hp.mass[:] = 0.0
        _say(f"[tier] {name} top_p={top_p}")
        out = decode_attend(g, q, lcd, pt, top_p=top_p, max_seq_len=c.max_len, tail=tailm, hp=hg)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref = oracle.decode(oc, c.orot, c.q, lc, c.pt, top_p, tail=otail, hp=hp)
        worst = 0.0
        for (b, h), r in ref.items():
            if lc[b] + ntail[b] == 0 and not np.any(hp.pos[b] >= 0):
                assert np.abs(out[b, h]).max() == 0.0
                continue
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (top_p, b, h, e)
        tm = np.zeros((B, 256, Hkv))
        oracle.add_mass(ref, tm, hp, c.wl.Hq)
        gm = tailm.mass.cpu().numpy().astype(np.float64)
        hm = hg.mass.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(gm, tm, rtol=1e-3, atol=1e-7)
        np.testing.assert_allclose(hm, hp.mass, rtol=1e-3, atol=1e-7)
        assert hp.mass.sum() > 0
        _say(f"[tier] {name} top_p={top_p} ok, worst rel err {worst:.2e}, tier mass {hp.mass.sum():.3f}")


@pytest.mark.parametrize("name,sketch", [("c3-gqa4-spikes-topp", None), ("c5-hadamard-topp", None),
                                         ("c3-gqa4-spikes-topp", 64)])
def test_hp_tier_update(name, sketch):
    """The promotion step against the oracle on caller-set masses (distinct values plus ties):
    tier positions, saved words, masses, binary16 rows and every key record bit-exact (also
    with 12-byte records of a 64-bit sketch, whose norm/correction word is word 2)."""
    from bit_kv_cache_compress_amd import Tail

    c = _case(name)
    dev = torch.device("cuda")
    B, Hkv, D, P = c.wl.B, c.wl.Hkv, c.wl.D, c.wl.P
    n = min(P, 128)
    lc = (c.lens - n).astype(np.int32)  # the last n tokens are the tail page just compressed
    oc, hp, g, hg = _tier_case(c, lc, 16, 41, sketch)
    rng = np.random.default_rng(42)
    hp.mass[:] = np.where(hp.pos >= 0, rng.random(hp.pos.shape).astype(np.float32), 0.0)
    tmass = rng.random((B, n, Hkv)).astype(np.float32) * 1.2
    tmass[:, 5:9] = tmass[:, 4:5]  # ties at one mass
    hg.mass.copy_(torch.from_numpy(hp.mass.astype(np.float32)))
    tail = Tail(B, n, Hkv, dev, mass=True)
    tk = np.stack([c.K[b, lc[b]:lc[b] + n] for b in range(B)]).astype(np.float16)
    tv = np.stack([c.V[b, lc[b]:lc[b] + n] for b in range(B)]).astype(np.float16)
    tail.k.copy_(torch.from_numpy(tk))
    tail.v.copy_(torch.from_numpy(tv))
    tail.len.fill_(n)
    tail.mass.copy_(torch.from_numpy(tmass))
    seq = torch.from_numpy(lc).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    hg.update(g, tail, n, seq, pt)
    torch.cuda.synchronize()
    oracle.hp_update(oc, hp, tk, tv, tmass, n, lc, c.pt)
    np.testing.assert_array_equal(hg.pos.cpu().numpy(), hp.pos.astype(np.int32))
    live = hp.pos >= 0
    np.testing.assert_array_equal(hg.saved.cpu().numpy().view(np.uint32)[live], hp.saved[live])
    np.testing.assert_array_equal(hg.mass.cpu().numpy()[live], hp.mass[live].astype(np.float32))
    np.testing.assert_array_equal(hg.k.cpu().numpy()[live].view(np.uint16), hp.k16[live].view(np.uint16))
    np.testing.assert_array_equal(hg.v.cpu().numpy()[live].view(np.uint16), hp.v16[live].view(np.uint16))
    np.testing.assert_array_equal(g.key_nc.cpu().numpy().view(np.uint32), oc.key_nc)
    np.testing.assert_array_equal(g.key_bits.cpu().numpy().view(np.uint32), oc.key_bits)
    entered = int(((hp.pos >= lc[:, None, None]) & live).sum())
    _say(f"[tier-update] {name} ok: {int(live.sum())} entries, {entered} entered from the tail")
    assert entered > 0


def test_hp_tier_pipeline():
    """Lazy updates with the high-precision tier: one token per step into the tail, a page
    compressed on a second stream, then the promotion and the retire; every 16th step's output
    against the oracle holding the same state (its own binary64 masses).  After each
    promotion the tier sets are compared; a different choice must still be valid under the
    oracle's masses (a near-tie decided by binary32 atomics), and ends the output checks."""
    from bit_kv_cache_compress_amd import HPTier, Tail, append, decode_attend

    c = _case("c3-gqa4-spikes-topp")
    dev = torch.device("cuda")
    B, Hkv, D, P, Hq = c.wl.B, c.wl.Hkv, c.wl.D, c.wl.P, c.wl.Hq
    C = 16
    L0 = 2 * P + 5
    steps = 2 * P + 9
    assert L0 + steps <= c.L
    ocache = oracle.PagedCache(c.npages, Hkv, P, D, c.wl.Gv)
    oracle.append(ocache, c.orot, c.K[:, :L0], c.V[:, :L0], np.zeros(B, np.int32), c.pt)
    g = upload(ocache, c)
    tail = Tail(B, 2 * P, Hkv, dev, mass=True)
    hg = HPTier(B, C, Hkv, dev)
    hp = oracle.HPTier(B, Hkv, C, D)
    tmass = np.zeros((B, 2 * P, Hkv))
    seq = torch.full((B,), L0, dtype=torch.int32, device=dev)
    pt = torch.from_numpy(c.pt).to(dev)
    q = torch.from_numpy(c.q).to(dev)
    side = torch.cuda.Stream()
    lc, nt, pending, comparing, promotions = L0, 0, None, True, 0
    for s in range(steps):
        t = L0 + s
        tail.append(torch.from_numpy(np.ascontiguousarray(c.K[:, t:t + 1])).to(dev),
                    torch.from_numpy(np.ascontiguousarray(c.V[:, t:t + 1])).to(dev))
        tmass[:, nt] = 0.0
        nt += 1
        if nt == P + 1 and pending is None:
            ev = torch.cuda.Event()
            ev.record()
            side.wait_event(ev)
            with torch.cuda.stream(side):
                for b in range(B):
                    kb, vb = tail.page(b, 0, P)
                    append(g, kb, vb, torch.tensor([lc], dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
                done = torch.cuda.Event()
                done.record()
            pending = (done, s + 4)
        if pending is not None and s == pending[1]:
            torch.cuda.current_stream().wait_event(pending[0])
            hg.update(g, tail, P, seq, pt)
            tail.retire(P, seq)
            if comparing:
                oracle.append(ocache, c.orot, c.K[:, lc:lc + P], c.V[:, lc:lc + P], np.full(B, lc, np.int32), c.pt)
                tk = c.K[:, lc:lc + P].astype(np.float16)
                tv = c.V[:, lc:lc + P].astype(np.float16)
                before = {(b, h): ({int(p): hp.mass[b, h, i] for i, p in enumerate(hp.pos[b, h]) if p >= 0},
                                   {lc + j: tmass[b, j, h] for j in range(P)}) for b in range(B) for h in range(Hkv)}
                oracle.hp_update(ocache, hp, tk, tv, tmass, P, np.full(B, lc, np.int32), c.pt)
                torch.cuda.synchronize()
                gpos = hg.pos.cpu().numpy()
                for b in range(B):
                    for h in range(Hkv):
                        want = {int(p) for p in hp.pos[b, h] if p >= 0}
                        got = {int(p) for p in gpos[b, h] if p >= 0}
                        if got != want:
                            allm = dict(before[(b, h)][0])
                            allm.update(before[(b, h)][1])
                            kth = sorted(allm.values(), reverse=True)[C - 1]
                            tol = 1e-3 * max(allm.values())
                            assert all(allm[p] >= kth - tol for p in got), (b, h)
                            comparing = False
                tmass = np.concatenate([tmass[:, P:], np.zeros_like(tmass[:, :P])], axis=1)
                promotions += 1
            lc, nt, pending = lc + P, nt - P, None
        out = decode_attend(g, q, seq, pt, top_p=c.wl.top_p, max_seq_len=c.L, tail=tail, hp=hg)
        if comparing:
            tk = np.zeros((B, 2 * P, Hkv, D), np.float16)
            tv = np.zeros_like(tk)
            tk[:, :nt] = c.K[:, lc:lc + nt].astype(np.float16)
            tv[:, :nt] = c.V[:, lc:lc + nt].astype(np.float16)
            ref = oracle.decode(ocache, c.orot, c.q, np.full(B, lc, np.int32), c.pt, c.wl.top_p,
                                tail=(tk, tv, np.full(B, nt, np.int32)), hp=hp)
            oracle.add_mass(ref, tmass, hp, Hq)
            if s % 16 == 0 or s == steps - 1:
                o = out.cpu().numpy()
                for (b, h), r in ref.items():
                    assert rel_err(o[b, h], r["out"]) <= TOL, (s, b, h)
                _say(f"[tier-lazy] step {s}: {lc} compressed + {nt} tail tokens, "
                     f"{int((hp.pos >= 0).sum())} tier entries ok")
    assert promotions >= 1
    torch.cuda.synchronize()
    _say(f"[tier-lazy] done, compared through the end: {comparing}")


@pytest.mark.parametrize("name", ["c1-full-fp32-dense", "c2-outliers-ragged", "c3-gqa4-spikes-topp",
                                  "c5-hadamard-topp", "gqa8-topp"])
def test_decode_with_fused_append(name):
    """A decode that appends the newest token of every sequence itself (its encoding rides in
    the query-preparation launch): cache bytes bit-exact against the oracle's, outputs within
    the bar, and both bit-identical to a separate append followed by a decode."""
    from bit_kv_cache_compress_amd import append, decode_attend
    from tests.kvc_testlib import gpu_empty_cache

    c = _case(name)
    assert np.all(c.lens >= 1)
    dev = torch.device("cuda")
    B = c.wl.B
    pt = torch.from_numpy(c.pt).to(dev)
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    last = c.lens.astype(np.int64) - 1
    k_new = torch.from_numpy(np.ascontiguousarray(c.K[np.arange(B), last][:, None])).to(dev)
    v_new = torch.from_numpy(np.ascontiguousarray(c.V[np.arange(B), last][:, None])).to(dev)
    start = torch.from_numpy(last.astype(np.int32)).to(dev)
    outs, caches = [], []
    for fused in (True, False):
        g = gpu_empty_cache(c)
        for b in range(B):
            n = int(c.lens[b]) - 1
            if n > 0:
                append(g, torch.from_numpy(np.ascontiguousarray(c.K[b:b + 1, :n])).to(dev),
                       torch.from_numpy(np.ascontiguousarray(c.V[b:b + 1, :n])).to(dev),
                       torch.zeros(1, dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
        if fused:
            out = decode_attend(g, q, lens, pt, top_p=c.wl.top_p, max_seq_len=c.max_len, append=(k_new, v_new, start))
        else:
            append(g, k_new, v_new, start, pt)
            out = decode_attend(g, q, lens, pt, top_p=c.wl.top_p, max_seq_len=c.max_len)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        caches.append(download(g))
    stats = compare_caches(caches[0], c.ocache, c)
    for key in caches[0]:
        np.testing.assert_array_equal(caches[0][key], caches[1][key])
    np.testing.assert_array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    ref = c.oracle_decode(c.ocache, c.wl.top_p)
    worst = max(float(rel_err(outs[0][b, h], r["out"])) for (b, h), r in ref.items())
    assert worst <= TOL
    _say(f"[fused-append] {name} ok {stats}, worst rel err {worst:.2e}")


def test_decode_with_fused_append_fallback():
    """More new token-heads than the fused launch takes (dense rotation, > 8192): the decode
    appends them with a launch of its own first.  Three copies of one sequence, 3 x 3096 new
    token-heads each step: bytes and outputs bit-identical to a separate append and decode,
    outputs within the bar of the oracle's."""
    from bit_kv_cache_compress_amd import KVCache, append, decode_attend

    c = _case("c1-full-fp32-dense")  # B = 1, Hkv = 1, 4096 tokens
    dev = torch.device("cuda")
    n0, R = 1000, 3
    n_new = int(c.lens[0]) - n0
    assert R * n_new * c.wl.Hkv > 8192
    pt3 = torch.from_numpy(np.stack([c.pt[0] + i * c.npages for i in range(R)]).astype(np.int32)).to(dev)
    K3 = np.repeat(c.K, R, axis=0)
    V3 = np.repeat(c.V, R, axis=0)
    kn = torch.from_numpy(np.ascontiguousarray(K3[:, n0:])).to(dev)
    vn = torch.from_numpy(np.ascontiguousarray(V3[:, n0:])).to(dev)
    start = torch.full((R,), n0, dtype=torch.int32, device=dev)
    q3 = torch.from_numpy(np.repeat(c.q, R, axis=0)).to(dev)
    lens3 = torch.full((R,), int(c.lens[0]), dtype=torch.int32, device=dev)
    outs, caches = [], []
    for fused in (True, False):
        g = KVCache(R * c.npages, 1, c.rot_raw, rot_kind=c.rot_kind, page_size=c.wl.P, value_group=c.wl.Gv, device=dev)
        append(g, torch.from_numpy(np.ascontiguousarray(K3[:, :n0])).to(dev),
               torch.from_numpy(np.ascontiguousarray(V3[:, :n0])).to(dev), torch.zeros(R, dtype=torch.int32, device=dev),
               pt3)
        if fused:
            out = decode_attend(g, q3, lens3, pt3, top_p=1.0, max_seq_len=c.max_len, append=(kn, vn, start))
        else:
            append(g, kn, vn, start, pt3)
            out = decode_attend(g, q3, lens3, pt3, top_p=1.0, max_seq_len=c.max_len)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        caches.append(download(g))
    for key in caches[0]:
        np.testing.assert_array_equal(caches[0][key], caches[1][key])
    np.testing.assert_array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    ref = c.oracle_decode(c.ocache, 1.0)[(0, 0)]["out"]
    for i in range(R):
        assert rel_err(outs[0][i, 0], ref) <= TOL
    _say("[fused-append] fallback ok")


@pytest.mark.parametrize("rot", ["dense", "hadamard"])
def test_degenerate_inputs(rot):
    """The method's degenerate cases against the oracle: a zero query (delta = 0, every code
    0, equal scores), zero keys (norm 0, correction 1), value groups of one value (scale 0),
    a sequence whose keys are all equal (one bin: Top-p keeps all of it), one-token and
    empty sequences, and Top-p at 1e-6 (the top bin only), 0.5, 0.999999 and 1."""
    from bit_kv_cache_compress_amd import append, decode_attend
    from tests.kvc_testlib import gpu_empty_cache

    wl = W.CONFIGS[2].scaled(B=5, Hq=8, Hkv=2, P=64, rot=rot)
    c = Case(wl, L=700, seq_lens=[700, 700, 1, 0, 333])
    rng = np.random.default_rng(77)
    c.q[0, 0] = 0.0                                    # zero query
    c.q[1, 3] = 2.5                                    # constant query
    c.K[0, rng.choice(700, 40, replace=False), 1] = 0  # zero keys
    c.K[1] = c.K[1, :1]                                # all keys of sequence 1 equal
    c.V[0, :, 0, 32:64] = 1.25                         # one value group constant
    c.V[4, :, 1] = 0.0                                 # zero values
    c.ocache = c.oracle_cache()
    dev = torch.device("cuda")
    g = gpu_empty_cache(c)
    pt = torch.from_numpy(c.pt).to(dev)
    for b in range(c.wl.B):
        n = int(c.lens[b])
        if n:
            append(g, torch.from_numpy(np.ascontiguousarray(c.K[b:b + 1, :n])).to(dev),
                   torch.from_numpy(np.ascontiguousarray(c.V[b:b + 1, :n])).to(dev),
                   torch.zeros(1, dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
    torch.cuda.synchronize()
    compare_caches(download(g), c.ocache, c)
    from bit_kv_cache_compress_amd import DecodeDebug
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    for top_p in (1e-6, 0.5, 0.999999, 1.0):
        dbg = DecodeDebug.allocate(c.wl.B, c.wl.Hq, c.max_len, top_p < 1.0, dev)
        out = decode_attend(g, q, lens, pt, top_p=top_p, max_seq_len=c.max_len, debug=dbg)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref = c.oracle_decode(c.ocache, top_p)
        for (b, h), r in ref.items():
            n = int(c.lens[b])
            np.testing.assert_array_equal(dbg.q_codes[b, h].cpu().numpy(), r["u"])
            if n == 0:
                assert np.abs(out[b, h]).max() == 0.0
                continue
            if top_p < 1.0:
                cnt = int(dbg.sel_count[b, h])
                np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            assert rel_err(out[b, h], r["out"]) <= TOL, (top_p, b, h)
        # equal keys: every token in one bin, so Top-p keeps them all
        if top_p < 1.0:
            assert int(dbg.sel_count[1, 0]) == 700
        _say(f"[degenerate] {rot} top_p={top_p} ok")
    assert np.all(ref[(0, 0)]["u"] == 0)


@pytest.mark.parametrize("name", ["c1-full-fp32-dense", "c2-outliers-ragged", "c3-gqa4-spikes-topp",
                                  "c4-paged-g64-ragged", "c5-hadamard-topp", "gqa2-pages16-p0.5", "gqa8-topp"])
def test_narrow_sketch(name):
    """A 64-bit key sketch (the first 64 rotated coordinates, 12-byte key records) against the
    oracle's: appended bytes bit-exact, the query codes and parameters, integer and binary32
    scores and Top-p sets bit-exact, outputs within the bar, at the case's Top-p and with
    full softmax (the matrix-core, dot8 and full-softmax score paths)."""
    c = _case(name)
    oc = c.oracle_cache(sketch=64)
    _say(f"[sketch] {name} append")
    g = gpu_append(c, sketch=64)
    stats = compare_caches(download(g), oc, c)
    assert g.keys.shape[-1] == 3
    for top_p in sorted({c.wl.top_p, 1.0}):
        out, dbg = _decode_with_debug(c, g, top_p)
        ref = c.oracle_decode(oc, top_p)
        qc, qp = dbg.q_codes.cpu().numpy(), dbg.q_params.cpu().numpy()
        A, S = dbg.iscores.cpu().numpy(), dbg.scores.cpu().numpy()
        worst = 0.0
        for (b, h), r in ref.items():
            np.testing.assert_array_equal(qc[b, h], r["u"])
            assert np.all(r["u"][64:] == 0)
            np.testing.assert_array_equal(qp[b, h], np.array([r["vl"], r["delta"], r["c0"], r["c1"]], np.float32))
            n = int(c.lens[b])
            np.testing.assert_array_equal(A[b, h, :n], r["A"])
            np.testing.assert_array_equal(S[b, h, :n].view(np.uint32), r["score"].view(np.uint32))
            if top_p < 1.0 and n > 0:
                cnt = int(dbg.sel_count[b, h])
                np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            if n == 0:
                assert np.abs(out[b, h]).max() == 0.0
                continue
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (top_p, b, h, e)
        # the fast path (no debug outputs) gives the same result
        out2, _ = _decode_with_debug(c, g, top_p, scores=False)
        np.testing.assert_array_equal(out2.view(np.uint32), out.view(np.uint32))
        _say(f"[sketch] {name} top_p={top_p} ok {stats}, worst rel err {worst:.2e}")
    if c.wl.top_p < 1.0:
        # binary16 keys: the sketch chooses the set, the softmax uses exact scores
        oe = c.oracle_cache(exact_keys=True, sketch=64)
        ge = upload(oe, c)
        out, _ = _decode_with_debug(c, ge, c.wl.top_p, scores=False)
        ref = c.oracle_decode(oe, c.wl.top_p)
        for (b, h), r in ref.items():
            if int(c.lens[b]) == 0:
                continue
            assert rel_err(out[b, h], r["out"]) <= TOL, ("exact", b, h)
        _say(f"[sketch] {name} exact scores ok")


@pytest.mark.parametrize("top_p", [0.9, 1.0])
def test_chunk_boundary_lengths(top_p):
    """Sequence lengths on both sides of the 512-token score chunks, the 1024-token attention
    chunks and the 256-token pages (masking of the last chunk, of the last histogram split
    and of the merge's chunk count), and a batch of empty sequences."""
    from bit_kv_cache_compress_amd import decode_attend

    lens = [1, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2049]
    wl = W.CONFIGS[2].scaled(B=len(lens), Hq=4, Hkv=1, P=256, top_p=top_p)
    c = Case(wl, L=max(lens), seq_lens=lens)
    c.ocache = c.oracle_cache()
    dev = torch.device("cuda")
    g = upload(c.ocache, c)
    q = torch.from_numpy(c.q).to(dev)
    lt = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    # four extra page-table columns (page 0, never reached) let a workspace be planned for
    # sequences longer than any present
    wide = np.concatenate([c.pt, np.zeros((c.pt.shape[0], 4), c.pt.dtype)], axis=1)
    pt = torch.from_numpy(wide).to(dev)
    for max_len in (c.max_len, wide.shape[1] * 256):
        out = decode_attend(g, q, lt, pt, top_p=top_p, max_seq_len=max_len)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        ref = c.oracle_decode(c.ocache, top_p)
        worst = 0.0
        for (b, h), r in ref.items():
            e = float(rel_err(out[b, h], r["out"]))
            worst = max(worst, e)
            assert e <= TOL, (max_len, lens[b], h, e)
        _say(f"[boundary] top_p={top_p} max_len={max_len} ok, worst rel err {worst:.2e}")
    # every sequence empty: zeros
    zero = torch.zeros_like(lt)
    out = decode_attend(g, q, zero, pt, top_p=top_p, max_seq_len=c.max_len)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0


def test_topp_dispatch_classes_poisoned_workspace():
    """Top-p heads of both dispatch classes of the attention pass (more, and at most, 64 kept
    tokens per 1024-token chunk), decoded on a workspace filled with 0xFF bytes (NaN as
    binary32): every partial that the merge reads is written by this call, whatever order
    the threshold pass gave the heads."""
    from bit_kv_cache_compress_amd import decode_attend, decode_workspace_bytes

    wl = W.CONFIGS[2].scaled(B=2, Hq=8, Hkv=2, P=256)
    c = Case(wl, L=16384)
    c.ocache = c.oracle_cache()
    ref = c.oracle_decode(c.ocache, wl.top_p)
    dense = {bh for bh, r in ref.items() if r["idx"].size * 1024 > 64 * int(c.lens[bh[0]])}
    assert 0 < len(dense) < len(ref), f"need heads of both classes, got {len(dense)} dense of {len(ref)}"
    dev = torch.device("cuda")
    g = upload(c.ocache, c)
    q = torch.from_numpy(c.q).to(dev)
    lt = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    ws = torch.full((decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, c.max_len, wl.top_p),), 255, dtype=torch.uint8,
                    device=dev)
    for rep in range(2):  # the second call runs on the first call's leftovers
        out = decode_attend(g, q, lt, pt, top_p=wl.top_p, max_seq_len=c.max_len, workspace=ws)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        for (b, h), r in ref.items():
            assert rel_err(out[b, h], r["out"]) <= TOL, (rep, b, h, (b, h) in dense)
    _say(f"[order] {len(dense)} dense heads of {len(ref)}: ok on a poisoned workspace")


@pytest.mark.parametrize("scores", [True, False])
def test_topp_many_heads_ragged(scores):
    """128 query heads (4 sequences of 32, enough heads for the one-kernel histogram and
    threshold pass) with ragged lengths and an empty sequence: top bins, thresholds, counts and
    index sets equal the oracle's bit for bit, outputs within the tolerance, twice in a row on
    one workspace; scores=True runs the debug score kernel, the other the matrix-core one."""
    wl = W.CONFIGS[2].scaled(B=4, Hq=32, Hkv=8, P=256)
    lens = [0, 1, 3001, 8192]
    c = Case(wl, L=max(lens), seq_lens=lens)
    c.ocache = c.oracle_cache()
    g = upload(c.ocache, c)
    ref = c.oracle_decode(c.ocache, wl.top_p)
    for rep in range(2):
        out, dbg = _decode_with_debug(c, g, wl.top_p, scores=scores)
        for (b, h), r in ref.items():
            n = int(c.lens[b])
            if n == 0:
                assert np.abs(out[b, h]).max() == 0.0 and int(dbg.sel_count[b, h]) == 0
                continue
            cnt = int(dbg.sel_count[b, h])
            assert cnt == len(r["idx"]), (rep, b, h, cnt, len(r["idx"]))
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            bins = dbg.sel_bins[b, h].cpu().numpy()
            assert (int(bins[0]), int(bins[1])) == (r["emax"], r["bstar"]), (b, h)
            assert rel_err(out[b, h], r["out"]) <= TOL, (rep, b, h)
    _say(f"[many heads] scores={scores} ok")


def test_topp_spans_small_pages():
    """16-token pages under spans of 4 attention chunks (a light head's wave over 4096 tokens
    reads 257 page ids, the most its LDS holds) and a ragged length that ends inside a span:
    sets and outputs against the oracle."""
    wl = W.CONFIGS[2].scaled(B=2, Hq=8, Hkv=2, P=16)
    lens = [9000, 4097]
    c = Case(wl, L=max(lens), seq_lens=lens)
    c.ocache = c.oracle_cache()
    g = upload(c.ocache, c)
    ref = c.oracle_decode(c.ocache, wl.top_p)
    light = sum(1 for (b, h), r in ref.items() if r["idx"].size * 4096 <= 64 * int(c.lens[b]))
    assert light > 0, "no head takes spans of 4 chunks"
    out, dbg = _decode_with_debug(c, g, wl.top_p, scores=False)
    for (b, h), r in ref.items():
        cnt = int(dbg.sel_count[b, h])
        np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
        assert rel_err(out[b, h], r["out"]) <= TOL, (b, h)
    _say(f"[small pages] {light} of {len(ref)} heads with spans of 4 chunks: ok")


def test_topp_long_sequence():
    """One 262144-token sequence at Top-p 0.95 (the ultra-long workload's rotation and page
    size; 8 query / 2 KV heads): 64 histogram splits per head, dense heads keeping 60-70% of
    their tokens (several batches per attention chunk) and 256 partial slots per head in the
    merge.  Index sets equal the oracle's bit for bit, outputs within the tolerance."""
    wl = W.CONFIGS[4].scaled(B=1, Hq=8, Hkv=2)
    c = Case(wl, L=262144)
    c.ocache = c.oracle_cache()
    g = upload(c.ocache, c)
    ref = c.oracle_decode(c.ocache, wl.top_p)
    out, dbg = _decode_with_debug(c, g, wl.top_p, scores=False)
    worst = 0.0
    for (b, h), r in ref.items():
        cnt = int(dbg.sel_count[b, h])
        assert cnt == len(r["idx"]), (b, h, cnt, len(r["idx"]))
        np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
        e = float(rel_err(out[b, h], r["out"]))
        worst = max(worst, e)
        assert e <= TOL, (b, h, e)
    _say(f"[long] 262144 tokens, top_p={wl.top_p}: ok, worst rel err {worst:.2e}")


@pytest.mark.parametrize("lens,variant", [([5000, 2300], "g32-p256"), ([1, 777], "g32-p256"),
                                          ([5000, 2300], "g64-p64"), ([4100, 3000], "sketch64"),
                                          ([3000, 2500, 1, 4100], "128heads")])
def test_topp_masked_groups(lens, variant):
    """Every head dense (the attention pass's block-per-KV-head numbering), the 4 query heads
    of KV head 0 each keeping about 90% of their tokens (the masked matrix-core pass over every
    record of a chunk) and those of KV head 1 some 15-25% (the per-head gather), in one call:
    ragged lengths that end inside a chunk, and blocks whose chunks lie past the end.  The
    variants cover the pass's builds: value groups of 32 and 64, pages of 256 and 64 tokens,
    the full and the 64-bit key sketch; and 128 heads over 4 sequences (the one-block histogram
    and threshold pass, an alternation of masked and gathered groups, a one-token sequence).
    Index sets equal the oracle's bit for bit, outputs within the tolerance, twice in a row on
    one workspace."""
    spec = {"g32-p256": dict(), "g64-p64": dict(Gv=64, P=64), "sketch64": dict(),
            "128heads": dict(B=4, Hq=32, Hkv=8)}[variant]
    wl = W.CONFIGS[4].scaled(**{**dict(B=2, Hq=8, Hkv=2), **spec})
    c = Case(wl, L=max(lens), seq_lens=lens)
    G = wl.Hq // wl.Hkv
    for kvh in range(wl.Hkv):  # even KV heads: flat softmax, most tokens kept; odd: a minority
        c.q[:, G * kvh:G * (kvh + 1)] *= 0.3 if kvh % 2 == 0 else (1.4 if variant == "sketch64" else 2.0)
    c.ocache = c.oracle_cache(sketch=64 if variant == "sketch64" else None)
    g = upload(c.ocache, c)
    ref = c.oracle_decode(c.ocache, wl.top_p)
    frac = {bh: r["idx"].size / int(c.lens[bh[0]]) for bh, r in ref.items()}
    if lens[0] > 1000:
        assert all(f * 1024 * 2 > 64 for f in frac.values()), frac  # every head dense
        assert all(frac[(b, h)] > 0.25 for b in range(wl.B) for h in range(4) if c.lens[b] > 0), frac
        assert any(min(frac[(b, h)] for h in range(4, 8)) <= 0.25 for b in range(wl.B) if c.lens[b] > 1), frac
    for rep in range(2):
        out, dbg = _decode_with_debug(c, g, wl.top_p, scores=False)
        for (b, h), r in ref.items():
            cnt = int(dbg.sel_count[b, h])
            assert cnt == len(r["idx"]), (rep, b, h, cnt, len(r["idx"]))
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
            assert rel_err(out[b, h], r["out"]) <= TOL, (rep, b, h, frac[(b, h)])
    _say(f"[masked] lens={lens} {variant}: ok")


def _random_case(i):
    """Seeded random geometry (its own input streams: workload index 100 + i)."""
    rng = np.random.default_rng(4242 + i)
    if i % 4 == 3:  # 128 query heads: the one-block histogram and threshold pass
        G, Hkv, B = 4, 8, 4
        L = int(rng.integers(300, 4000))
    else:
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]) if G == 8 else rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 4))
        L = int(rng.integers(300, 12000))
    P = int(rng.choice([16, 64, 128, 256]))
    Gv = int(rng.choice([32, 64]))
    rot = str(rng.choice(["dense", "hadamard"]))
    top_p = float(rng.choice([0.5, 0.8, 0.95, 1.0]))
    spike = float(rng.choice([0.0, 0.01]))
    sketch = int(rng.choice([128, 64]))
    lens = [int(x) for x in rng.integers(0, L + 1, size=B)]
    lens[0] = L
    if B > 1 and i % 3 == 0:
        lens[-1] = int(rng.choice([0, 1]))  # an empty or one-token sequence
    wl = W.CONFIGS[2].scaled(name=f"random-{i}", index=100 + i, B=B, Hq=G * Hkv, Hkv=Hkv, L=L, P=P, Gv=Gv, rot=rot,
                             top_p=top_p, spike_frac=spike, shuffle_pages=bool(rng.integers(0, 2)))
    return wl, lens, sketch


@pytest.mark.parametrize("i", range(32))
def test_random_geometry(i):
    """Seeded random geometries (GQA groups 1-8, 1-4 sequences of up to 12000 tokens with
    random lengths including empty and one-token ones, 128 query heads in every fourth case,
    pages of 16-256 tokens, value groups 32/64, both rotations, Top-p 0.5-0.95 or
    full softmax, with or without spikes, 128- or 64-bit sketches, shuffled pages): the append's
    bytes against the oracle's encoding, then the decode over the oracle's cache bytes (sets
    bit-exact, outputs within the tolerance)."""
    wl, lens, sketch = _random_case(i)
    sk = None if sketch == 128 else sketch
    c = Case(wl, L=max(lens), seq_lens=lens)
    c.ocache = c.oracle_cache(sketch=sk)
    g_app = gpu_append(c, sketch=sk)
    stats = compare_caches(download(g_app), c.ocache, c)
    g = upload(c.ocache, c)
    ref = c.oracle_decode(c.ocache, wl.top_p)
    out, dbg = _decode_with_debug(c, g, wl.top_p, scores=False, dist=False)
    worst = 0.0
    for (b, h), r in ref.items():
        n = int(c.lens[b])
        if n == 0:
            assert np.abs(out[b, h]).max() == 0.0, (b, h)
            continue
        if wl.top_p < 1.0:
            cnt = int(dbg.sel_count[b, h])
            assert cnt == len(r["idx"]), (i, b, h, cnt, len(r["idx"]))
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
        e = float(rel_err(out[b, h], r["out"]))
        worst = max(worst, e)
        assert e <= TOL, (i, b, h, e)
    _say(f"[random {i}] G={wl.Hq // wl.Hkv} Hkv={wl.Hkv} B={wl.B} lens={lens} P={wl.P} Gv={wl.Gv} {wl.rot} "
         f"top_p={wl.top_p} sketch={sketch}: ok {stats}, worst {worst:.1e}")
