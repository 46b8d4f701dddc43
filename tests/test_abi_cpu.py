"""C ABI checks that need no GPU: the library loads, exports every function that
include/kv_compress.h declares, and rejects bad arguments on the host (negative code and a
message, before any HIP call)."""
import ctypes
import os
import re

import pytest

from bit_kv_cache_compress_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def _declared():
    src = open(os.path.join(ROOT, "include", "kv_compress.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = _declared()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kv_version() == 10000


def _desc(**kw):
    d = dict(head_dim=128, num_kv_heads=8, value_group=32, page_size=256, num_pages=16, rot_kind=0,
             rot=0x10000, keys=0x10000, vals=0x10000, keys_f16=None, key_center=None, sketch_dim=0)
    d.update(kw)
    return L.KVCacheDesc(*[d[f] for f, _ in L.KVCacheDesc._fields_])


def _decode(desc, B=2, Hq=32, max_seq_len=1000, max_pages=4, top_p=1.0, ws_bytes=None, q=FAKE, out=FAKE):
    if ws_bytes is None:
        ws_bytes = L.lib().kv_decode_workspace_bytes(B, Hq, desc.num_kv_heads, max_seq_len, 128, top_p)
    return L.lib().kv_decode_attend(ctypes.byref(desc), q, B, Hq, FAKE, max_seq_len, FAKE, max_pages, top_p, out,
                                    None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), L.KV_ERR_UNSUPPORTED),
    (dict(value_group=16), L.KV_ERR_UNSUPPORTED),
    (dict(page_size=100), L.KV_ERR_UNSUPPORTED),
    (dict(page_size=8), L.KV_ERR_UNSUPPORTED),
    (dict(num_pages=0), L.KV_ERR_ARG),
    (dict(num_pages=1 << 24), L.KV_ERR_UNSUPPORTED),  # 2^35 slots: above the 32-bit slot index
    (dict(num_kv_heads=0), L.KV_ERR_ARG),
    (dict(rot_kind=7), L.KV_ERR_ARG),
    (dict(keys=0), L.KV_ERR_ARG),
    (dict(keys_f16=0x10008), L.KV_ERR_ARG),  # binary16 keys not 16-byte aligned
    (dict(key_center=0x10004), L.KV_ERR_ARG),  # key centers not 16-byte aligned
    (dict(sketch_dim=96), L.KV_ERR_UNSUPPORTED),  # sketch widths are 128 and 64
    (dict(vals=0), L.KV_ERR_ARG),
    (dict(rot=0), L.KV_ERR_ARG),
])
def test_bad_cache_descriptor(kw, code):
    assert _decode(_desc(**kw)) == code
    assert L.last_error()
    rc = L.lib().kv_compress_append(ctypes.byref(_desc(**kw)), 0, FAKE, FAKE, 1, 4, FAKE, FAKE, 1, None)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), L.KV_ERR_ARG),
    (dict(Hq=12), L.KV_ERR_ARG),        # not a multiple of Hkv = 8
    (dict(Hq=24), L.KV_ERR_UNSUPPORTED),  # group 3
    (dict(Hq=128), L.KV_ERR_UNSUPPORTED),  # group 16
    (dict(max_seq_len=0), L.KV_ERR_ARG),
    (dict(max_seq_len=5000, max_pages=4), L.KV_ERR_ARG),  # pages cover only 1024 tokens
    (dict(top_p=0.0), L.KV_ERR_ARG),
    (dict(top_p=-0.5), L.KV_ERR_ARG),
    (dict(top_p=float("nan")), L.KV_ERR_ARG),
    (dict(B=1 << 19, Hq=32, top_p=0.9), L.KV_ERR_UNSUPPORTED),  # more sequences than the grid holds
    (dict(B=70000, Hq=32, top_p=1.0), L.KV_ERR_UNSUPPORTED),
    (dict(q=None), L.KV_ERR_ARG),
    (dict(out=None), L.KV_ERR_ARG),
])
def test_bad_decode_arguments(kw, code):
    ws = kw.pop("ws_bytes", 1 << 30)
    assert _decode(_desc(), ws_bytes=ws, **kw) == code
    assert L.last_error()


def test_workspace_too_small():
    need = L.lib().kv_decode_workspace_bytes(2, 32, 8, 1000, 128, 0.9)
    assert need > 0
    assert _decode(_desc(), top_p=0.9, ws_bytes=need - 1) == L.KV_ERR_WORKSPACE
    assert "workspace" in L.last_error()
    tneed = L.lib().kv_topp_workspace_bytes(2, 32, 1000)
    rc = L.lib().kv_topp_select(FAKE, 1000, FAKE, 2, 32, 128, 0.9, FAKE, FAKE, FAKE, tneed - 1, None)
    assert rc == L.KV_ERR_WORKSPACE


def _struct_fields(name):
    src = open(os.path.join(ROOT, "include", "kv_compress.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    body = re.search(r"typedef struct " + name + r"\s*\{(.*?)\}\s*" + name + ";", src, flags=re.S).group(1)
    return [re.findall(r"(\w+)\s*(?:\[\w*\])?$", d.strip())[0] for d in body.split(";") if d.strip()]


@pytest.mark.parametrize("name,cls", [("kv_cache", "KVCacheDesc"), ("kv_debug", "KVDebug"), ("kv_tail", "KVTailDesc"),
                                      ("kv_hp", "KVHpDesc"), ("kv_decode_opts", "KVDecodeOpts")])
def test_binding_structs_match_header(name, cls):
    """The ctypes structures declare the header's members in the header's order."""
    assert [f for f, _ in getattr(L, cls)._fields_] == _struct_fields(name)


def test_workspace_sizes():
    lib = L.lib()
    assert lib.kv_workspace_bytes(4, 32, 8, 131072, 128, 0.9) == lib.kv_decode_workspace_bytes(4, 32, 8, 131072, 128,
                                                                                              0.9)
    full = lib.kv_decode_workspace_bytes(4, 32, 8, 131072, 128, 1.0)
    topp = lib.kv_decode_workspace_bytes(4, 32, 8, 131072, 128, 0.9)
    assert 0 < full < topp
    # the Top-p workspace holds at least a 16-bit bin distance per (sequence, head, token)
    assert topp >= 4 * 32 * 131072 * 2
    assert lib.kv_decode_workspace_bytes(4, 32, 8, 131072, 64, 0.9) == 0
    assert lib.kv_decode_workspace_bytes(0, 32, 8, 131072, 128, 0.9) == 0
    assert lib.kv_topp_workspace_bytes(1, 1, 0) == 0


@pytest.mark.parametrize("p", [0.0, 1.0, 1.5, -1.0, float("nan")])
def test_topp_select_rejects_p(p):
    rc = L.lib().kv_topp_select(FAKE, 100, FAKE, 1, 1, 128, p, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == L.KV_ERR_ARG


def test_append_argument_errors():
    lib = L.lib()
    d = _desc()
    assert lib.kv_compress_append(ctypes.byref(d), 2, FAKE, FAKE, 1, 4, FAKE, FAKE, 1, None) == L.KV_ERR_ARG
    assert lib.kv_compress_append(ctypes.byref(d), 0, None, FAKE, 1, 4, FAKE, FAKE, 1, None) == L.KV_ERR_ARG
    assert lib.kv_compress_append(ctypes.byref(d), 0, FAKE, FAKE, 0, 4, FAKE, FAKE, 1, None) == L.KV_ERR_ARG
    assert lib.kv_compress_append(ctypes.byref(d), 0, FAKE, FAKE, 1, -1, FAKE, FAKE, 1, None) == L.KV_ERR_ARG
    # zero new tokens is a no-op
    assert lib.kv_compress_append(ctypes.byref(d), 0, None, None, 1, 0, None, None, 1, None) == L.KV_OK
    assert lib.kv_compress_append(None, 0, FAKE, FAKE, 1, 4, FAKE, FAKE, 1, None) == L.KV_ERR_ARG


def _decode_tail(tail, desc=None, B=2, Hq=32, max_seq_len=1000, max_pages=4, top_p=1.0):
    desc = desc or _desc()
    ws = L.lib().kv_decode_workspace_bytes(B, Hq, desc.num_kv_heads, max_seq_len, 128, top_p)
    return L.lib().kv_decode_attend_tail(ctypes.byref(desc), ctypes.byref(tail) if tail is not None else None,
                                         FAKE, B, Hq, FAKE, max_seq_len, FAKE, max_pages, top_p, FAKE, None, FAKE,
                                         ws, None)


@pytest.mark.parametrize("kw", [dict(k=None), dict(v=None), dict(len=None), dict(capacity=0),
                                dict(k=0x10008)])
def test_bad_tail_descriptor(kw):
    d = dict(k=0x10000, v=0x10000, len=0x10000, capacity=256, mass=None)
    d.update(kw)
    tail = L.KVTailDesc(*[d[f] for f, _ in L.KVTailDesc._fields_])
    assert _decode_tail(tail) == L.KV_ERR_ARG
    assert L.last_error()


def test_null_tail_descriptor():
    assert _decode_tail(None) == L.KV_ERR_ARG


def _decode_ex(opts, desc=None, B=2, Hq=32, max_seq_len=1000, max_pages=4, top_p=1.0):
    desc = desc or _desc()
    ws = L.lib().kv_decode_workspace_bytes(B, Hq, desc.num_kv_heads, max_seq_len, 128, top_p)
    return L.lib().kv_decode_attend_ex(ctypes.byref(desc) if desc is not None else None,
                                       ctypes.byref(opts) if opts is not None else None, FAKE, B, Hq, FAKE,
                                       max_seq_len, FAKE, max_pages, top_p, FAKE, None, FAKE, ws, None)


def test_decode_ex_rejects_bad_options():
    """kv_decode_attend_ex: a misaligned dither, an invalid tail in the options and a bad
    cache descriptor are errors caught on the host."""
    assert _decode_ex(L.KVDecodeOpts(None, 0x10002, None)) == L.KV_ERR_ARG
    assert "q_dither" in L.last_error()
    bad_tail = L.KVTailDesc(0x10000, 0x10000, None, 256, None)
    assert _decode_ex(L.KVDecodeOpts(ctypes.pointer(bad_tail), None, None)) == L.KV_ERR_ARG
    assert _decode_ex(L.KVDecodeOpts(None, None, None), desc=_desc(head_dim=64)) == L.KV_ERR_UNSUPPORTED
    assert _decode_ex(L.KVDecodeOpts(None, None, None), B=0) == L.KV_ERR_ARG
    rc = L.lib().kv_decode_attend_ex(None, None, FAKE, 2, 32, FAKE, 1000, FAKE, 4, 1.0, FAKE, None, FAKE, 1 << 30,
                                     None)
    assert rc == L.KV_ERR_ARG


def _hp(**kw):
    d = dict(k=0x10000, v=0x10000, pos=0x10000, saved=0x10000, mass=0x10000, capacity=64)
    d.update(kw)
    return L.KVHpDesc(*[d[f] for f, _ in L.KVHpDesc._fields_])


@pytest.mark.parametrize("kw", [dict(k=None), dict(pos=None), dict(saved=None), dict(mass=None),
                                dict(capacity=0), dict(capacity=1025), dict(v=0x10008), dict(mass=0x10002)])
def test_bad_tier_descriptor(kw):
    assert _decode_ex(L.KVDecodeOpts(None, None, ctypes.pointer(_hp(**kw)))) == L.KV_ERR_ARG
    assert L.last_error()


def test_tier_with_tail_needs_the_tail_mass():
    tail = L.KVTailDesc(0x10000, 0x10000, 0x10000, 256, None)
    assert _decode_ex(L.KVDecodeOpts(ctypes.pointer(tail), None, ctypes.pointer(_hp()))) == L.KV_ERR_ARG
    assert "mass" in L.last_error()


def test_hp_update_rejects_bad_arguments():
    lib = L.lib()
    tail = L.KVTailDesc(0x10000, 0x10000, 0x10000, 256, 0x10000)
    nomass = L.KVTailDesc(0x10000, 0x10000, 0x10000, 256, None)
    d, hp = _desc(), _hp()

    def upd(desc=d, h=hp, t=tail, B=2, n=256, seq=FAKE, pt=FAKE, mp=4):
        return lib.kv_hp_update(ctypes.byref(desc) if desc is not None else None,
                                ctypes.byref(h) if h is not None else None, ctypes.byref(t) if t is not None else None,
                                B, n, seq, pt, mp, None)
    assert upd(h=None) == L.KV_ERR_ARG
    assert upd(t=None) == L.KV_ERR_ARG
    assert upd(t=nomass) == L.KV_ERR_ARG
    assert upd(n=257) == L.KV_ERR_ARG                      # more than the tail holds
    assert upd(h=_hp(capacity=900), n=200) == L.KV_ERR_ARG  # more than 1024 candidates
    assert upd(seq=None) == L.KV_ERR_ARG
    assert upd(mp=0) == L.KV_ERR_ARG
    assert upd(desc=_desc(value_group=16)) == L.KV_ERR_UNSUPPORTED
    assert upd(n=0) == L.KV_OK



def test_noalloc_rejects_workspaces_above_its_static_array():
    """kv_decode_attend_noalloc has a 64 MiB static workspace per device: a decode that needs
    more is refused on the host (KV_ERR_WORKSPACE, nothing enqueued), as are bad shapes."""
    lib = L.lib()
    d = _desc(num_pages=4096)
    need = lib.kv_decode_workspace_bytes(4, 32, 8, 262144, 128, 0.9)
    assert need > 64 << 20
    rc = lib.kv_decode_attend_noalloc(ctypes.byref(d), None, FAKE, 4, 32, FAKE, 262144, FAKE, 1024, 0.9, FAKE, None,
                                      None)
    assert rc == L.KV_ERR_WORKSPACE and "static workspace" in L.last_error()
    rc = lib.kv_decode_attend_noalloc(ctypes.byref(d), None, FAKE, 4, 24, FAKE, 1000, FAKE, 4, 0.9, FAKE, None, None)
    assert rc == L.KV_ERR_UNSUPPORTED
