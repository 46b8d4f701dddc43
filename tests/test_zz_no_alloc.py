"""kv_decode_attend_noalloc (the decode whose workspace is the library's static per-device
array, for callers that cannot allocate) against kv_decode_attend_ex with a caller workspace:
bit-identical outputs and Top-p sets on two calls in a row, the second with a smaller input,
under Top-p and with full softmax, and with new tokens appended inside the call."""
import sys

import numpy as np
import pytest

import workloads as W
from tests.kvc_testlib import Case, gpu_append

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(c, g, top_p, noalloc, append=False):
    import bit_kv_cache_compress_amd as kvc

    dev = torch.device("cuda")
    q = torch.from_numpy(c.q).to(dev)
    lens = torch.from_numpy(c.lens).to(dev)
    pt = torch.from_numpy(c.pt).to(dev)
    dbg = kvc.DecodeDebug.allocate(c.wl.B, c.wl.Hq, c.max_len, top_p < 1.0, dev, scores=False)
    app = None
    if append:  # re-append the last token of every sequence inside the call
        last = torch.from_numpy(c.lens.astype(np.int64) - 1).to(dev)
        ar = torch.arange(c.wl.B, device=dev)
        K = torch.from_numpy(c.K).to(dev)
        V = torch.from_numpy(c.V).to(dev)
        app = (K[ar, last].unsqueeze(1).contiguous(), V[ar, last].unsqueeze(1).contiguous(),
               (lens - 1).contiguous())
    out = torch.full((c.wl.B, c.wl.Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    kvc.decode_attend(g, q, lens, pt, top_p=top_p, max_seq_len=c.max_len, out=out, debug=dbg, noalloc=noalloc,
                      append=app)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dbg


@pytest.mark.parametrize("top_p", [0.9, 1.0])
def test_noalloc_matches_workspace_decode(top_p):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = Case(W.CONFIGS[2].scaled(B=2, Hq=8, Hkv=2, P=128), L=6000)
    small = Case(W.CONFIGS[2].scaled(B=1, Hq=4, Hkv=1, P=64), L=1100)
    for name, c, append in (("first", big, False), ("second, smaller", small, True)):
        g = gpu_append(c)
        ref, dref = _run(c, g, top_p, noalloc=False, append=append)
        out, dout = _run(c, g, top_p, noalloc=True, append=append)
        assert np.isfinite(out).all()
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32)), name
        if top_p < 1.0:
            assert torch.equal(dout.sel_count, dref.sel_count)
            assert torch.equal(dout.sel_idx, dref.sel_idx)
            assert torch.equal(dout.sel_bins, dref.sel_bins)
        _say(f"[noalloc] top_p={top_p} {name} call (B={c.wl.B}, Hq={c.wl.Hq}, L={c.L}): identical")
