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

import workloads as W
from tests.kvc_testlib import Case, compare_caches, download, gpu_append, rel_err, upload

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


def _decode_with_debug(c, cache, top_p, scores=True, proxy=False):
    """Decode with debug outputs; scores=False runs the kernels of a decode without debug
    output (the per-token scores are not written) and still returns the Top-p sets."""
    from bit_kv_cache_compress_amd import DecodeDebug, decode_attend

    dev = torch.device("cuda")
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens.astype(np.int32)).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    dbg = DecodeDebug.allocate(c.wl.B, c.wl.Hq, c.max_len, top_p < 1.0, dev, scores=scores)
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
    same = all(np.array_equal(v, getattr(c.ocache, k)) for k, v in download(g).items())
    out, dbg = _decode_with_debug(c, g, c.wl.top_p, scores=False)
    ref = c.oracle_decode(c.ocache, c.wl.top_p)
    worst = max(float(rel_err(out[b, h], r["out"])) if int(c.lens[b]) else 0.0 for (b, h), r in ref.items())
    assert worst <= TOL
    if same and c.wl.top_p < 1.0:
        for (b, h), r in ref.items():
            cnt = int(dbg.sel_count[b, h])
            np.testing.assert_array_equal(dbg.sel_idx[b, h, :cnt].cpu().numpy(), r["idx"])
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
