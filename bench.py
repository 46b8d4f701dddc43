#!/usr/bin/env python3
"""Decode-step benchmark of the compressed-KV attention library on one MI355X.

A step is the whole decode hot path for one batch: append the newest token of every
sequence (key sign bits + norm/correction, 4-bit values) into the paged cache, then one
decode attention over every cached token (query rotation and int4 codes, binary x INT4
proxy scores, adaptive Top-p when the workload uses it, softmax and 4-bit value sums, merge).

Default workload: 32 query / 8 KV heads, head_dim 128, batch 4, 131072-token context, fp16
K/V N(0,1) with 1% query-correlated "spike" tokens, dense random rotation, value group 32,
256-token pages, adaptive Top-p 0.9.  The cache is filled before timing (inputs resident
in HBM); L2 and the 256 MB Infinity Cache are flushed between steps outside the timed
events.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode: KV tokens*heads attended/s and % of MI355X HBM peak"
APPEND_METRIC = "compressed-KV append: token-heads compressed/s and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
# Algorithmic bytes (the least a step must move): a cached key is 16 B of sign words + a 4 B
# norm/correction word per token-KV-head, read once per step; a cached value is 64 B of 4-bit
# codes + a 4 B scale/zero word per group, read once per attended token-KV-head (under Top-p:
# the union of the kept tokens of the KV head's query heads).  The design also moves a 2 B
# bin distance per (token, query head) (written by the score pass, read by the histogram and
# attention passes) and re-reads the key records of kept tokens; those count as design
# bytes, not algorithmic ones.
DIST_BYTES = 2


def value_bytes(Gv):
    return 64 + 4 * (128 // Gv)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload index 0..4 (default 2: GQA 128k Top-p)")
    ap.add_argument("--top-p", type=float, default=None,
                    help="override the workload's top_p (1 = full softmax, e.g. --config 2 --top-p 1: the "
                         "128k streaming check)")
    ap.add_argument("--append", action="store_true",
                    help="time the prefill append of workload 4 (32768 tokens x 32 KV heads, randomized "
                         "Hadamard rotation) instead of a decode step: token-heads compressed/s")
    ap.add_argument("--append-rotation", choices=("hadamard", "dense"), default="hadamard",
                    help="with --append: the rotation (dense: a seeded Haar rotation in binary16)")
    ap.add_argument("--no-flush", action="store_true", help="keep caches warm between steps")
    ap.add_argument("--lazy", action="store_true",
                    help="lazy updates: new tokens go to a binary16 tail, whole pages are compressed on a "
                         "second stream; times one page cycle (steps default to the page size)")
    ap.add_argument("--hp-capacity", type=int, default=0, metavar="C",
                    help="with --lazy: a high-precision tier of C binary16 entries per (sequence, KV head), "
                         "filled at each page compression by accumulated attention mass")
    ap.add_argument("--separate-append", action="store_true",
                    help="append the step's new tokens with a call of their own instead of inside the decode")
    ap.add_argument("--sketch-dim", type=int, default=128, choices=(128, 64),
                    help="sign bits per key: 128, or a narrow 64-bit sketch (12-byte key records)")
    ap.add_argument("--center-keys", action="store_true",
                    help="estimator variant: per-head key centers (the mean of the prefill keys)")
    ap.add_argument("--stochastic-query", action="store_true",
                    help="estimator variant: seeded stochastic rounding of the int4 query")
    ap.add_argument("--exact-keys", action="store_true",
                    help="also keep binary16 keys; Top-p attends the selected tokens with exact scores")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step (its kernels, on one stream) in a HIP graph once and time its "
                         "replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many steps after setup (for rocprofv3), no JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (a known-size kernel that "
                         "calibrates the FETCH_SIZE/WRITE_SIZE counters), no JSON")
    a = ap.parse_args()
    a.steps_given = a.steps is not None
    if a.steps is None:
        a.steps = 50
    return a


def workload(args):
    """The workload of --config, with --top-p applied (and named after it)."""
    import workloads as W

    wl = W.CONFIGS[args.config]
    if args.top_p is not None and args.top_p != wl.top_p:
        base = wl.name.rsplit("-topp", 1)[0] if wl.top_p < 1.0 else wl.name
        wl = wl.scaled(top_p=args.top_p, name=base + ("-full" if args.top_p >= 1.0 else f"-topp{args.top_p:g}"))
    return wl


def run_lazy(args):
    """Decode steps with lazy updates: each step writes the new token of every sequence into
    the binary16 tail and decodes over cache plus tail; when a tail holds more than a page, its
    first page is compressed into the cache on a second stream and retired 4 steps later.
    The timed region is one page cycle (page_size steps, one compression per sequence)."""
    import numpy as np
    import torch

    import bit_kv_cache_compress_amd as kvc
    import workloads as W

    wl = workload(args)
    if wl.len_range is not None:
        raise SystemExit("--lazy needs a workload with equal sequence lengths")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    D, Hq, Hkv, B, P, Gv, L = wl.D, wl.Hq, wl.Hkv, wl.B, wl.P, wl.Gv, wl.L
    steps = args.steps if args.steps_given else P
    total = args.warmup + steps
    # compressed tokens before the first step: whole pages, the rest (1 .. P tokens) in the tail;
    # the tail then passes P tokens at steps 0, P, 2P, ... so every window of P steps after the
    # first compresses one page per sequence
    Lc0 = (L - 1) // P * P
    T0 = L - Lc0
    log(f"[bench] lazy updates on {wl.name}: B={B} Hq={Hq} Hkv={Hkv} L={L} top_p={wl.top_p}; "
        f"{Lc0} compressed + {T0} tail tokens, {total} steps of one token")
    K, V, q = W.draw_device(wl, dev, L=L)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed(99))
    kvt = torch.float16 if wl.kv_dtype == "f16" else torch.float32
    KN = torch.randn((total, B, 1, Hkv, D), generator=g, device=dev).to(kvt)
    VN = torch.randn((total, B, 1, Hkv, D), generator=g, device=dev).to(kvt)
    pt_np, npages = W.page_layout(wl, np.full(B, L, np.int32), reserve=total + P)
    kind, rot = W.draw_rotation(wl)
    cache = kvc.KVCache(npages, Hkv, rot, rot_kind=kind, page_size=P, value_group=Gv, device=dev)
    pt = torch.from_numpy(pt_np).to(dev)
    kvc.append(cache, K[:, :Lc0].to(kvt).contiguous(), V[:, :Lc0].to(kvt).contiguous(),
               torch.zeros(B, dtype=torch.int32, device=dev), pt)
    C = args.hp_capacity
    tail = kvc.Tail(B, 2 * P, Hkv, dev, mass=C > 0)
    tail.append(K[:, Lc0:].to(kvt).contiguous(), V[:, Lc0:].to(kvt).contiguous())
    hp = kvc.HPTier(B, C, Hkv, dev) if C > 0 else None
    del K, V
    seq = torch.full((B,), Lc0, dtype=torch.int32, device=dev)
    Lmax = L + total
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvc.decode_workspace_bytes(B, Hq, Hkv, Lmax, wl.top_p), dtype=torch.uint8, device=dev)
    flush_buf = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)  # summed in its own dtype: reads only
    side = torch.cuda.Stream()
    st = dict(lc=Lc0, nt=T0, pending=None, compressions=0)
    starts = [torch.tensor([0], dtype=torch.int32, device=dev) for _ in range(B)]
    pts = [pt[b:b + 1].contiguous() for b in range(B)]

    def step(i):
        tail.append(KN[i], VN[i])
        st["nt"] += 1
        if st["nt"] == P + 1 and st["pending"] is None:
            ev = torch.cuda.Event()
            ev.record()
            side.wait_event(ev)
            with torch.cuda.stream(side):
                for b in range(B):
                    starts[b].fill_(st["lc"])
                    kb, vb = tail.page(b, 0, P)
                    kvc.append(cache, kb, vb, starts[b], pts[b])
                done = torch.cuda.Event()
                done.record()
            st["pending"] = (done, i + 4)
            st["compressions"] += 1
        if st["pending"] is not None and i == st["pending"][1]:
            torch.cuda.current_stream().wait_event(st["pending"][0])
            if hp is not None:
                hp.update(cache, tail, P, seq, pt)
            tail.retire(P, seq)
            st["lc"] += P
            st["nt"] -= P
            st["pending"] = None
        kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=st["lc"], out=out, workspace=ws, tail=tail,
                          hp=hp)

    for i in range(args.warmup):
        flush_buf.sum()
        step(i)
    torch.cuda.synchronize()
    c0 = st["compressions"]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    toks = []
    wall0 = time.perf_counter()
    for j in range(steps):
        flush_buf.sum()
        ev[j][0].record()
        step(args.warmup + j)
        ev[j][1].record()
        toks.append(st["lc"] + st["nt"])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms = statistics.mean(step_ms)
    value = statistics.mean(t * B * Hkv for t in toks) / (ms / 1e3)
    if hp is not None:
        log(f"[bench] tier: {int((hp.pos >= 0).sum())} entries filled, mass {float(hp.mass.sum()):.2f}")
    log(f"[bench] lazy step {ms * 1e3:.1f} us (median {statistics.median(step_ms) * 1e3:.1f}, "
        f"max {max(step_ms) * 1e3:.1f}); {value:.3e} KV token-heads/s; "
        f"{st['compressions'] - c0} page compressions on the second stream")
    result = {
        "metric": METRIC, "value": value, "unit": "KV token-heads/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i32 (1-bit x int4 popcount) + f32", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": L,
                   "head_dim": D, "top_p": wl.top_p, "value_group": Gv, "page_size": P, "rotation": wl.rot,
                   "kv_dtype": wl.kv_dtype, "lazy": True, "tail_tokens_at_start": T0, "hp_capacity": C,
                   "step": "append 1 token per sequence to the binary16 tail + decode over cache and tail; "
                           "a full page compressed on a second stream",
                   "cache_flushed_between_steps": True},
        "roofline": None, "cpu_baseline": None,
        "page_compressions_timed": st["compressions"] - c0,
        "step_us_median": round(statistics.median(step_ms) * 1e3, 2),
        "wall_ms_per_step_incl_flush": round(wall / steps * 1e3, 3),
    }
    print(json.dumps(result), flush=True)


def run_append(args):
    """The prefill append of workload 4: 32768 new tokens x 32 KV heads of binary16 K/V
    (N(0,1)) encoded with the randomized Hadamard rotation into the paged cache (sign bits,
    norm and correction of every key; 4-bit codes with scale and zero point of every value).
    One launch per step, timed with events on the stream it runs on; caches flushed between
    steps.  Algorithmic bytes: the K and V read (512 B per token-head) and the 20 B key and
    80 B value records written."""
    import numpy as np
    import torch

    import bit_kv_cache_compress_amd as kvc
    import workloads as W

    wl = W.CONFIGS[4]
    if args.append_rotation == "dense":
        wl = wl.scaled(rot="dense")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    D, P, Gv = wl.D, wl.P, wl.Gv
    n_new, Ha = wl.append_tokens, wl.append_heads
    name = f"{wl.rot}-append{n_new // 1024}k-{Ha}kvh-f16"
    log(f"[bench] append workload {name}: {n_new} tokens x {Ha} KV heads, rotation {wl.rot}, value group {Gv}")
    K, V, _ = W.draw_device(wl, dev, L=n_new, Hkv=Ha)
    pt_np, npages = W.page_layout(wl.scaled(Hkv=Ha), np.array([n_new], np.int32))
    kind, rot = W.draw_rotation(wl)
    cache = kvc.KVCache(npages, Ha, rot, rot_kind=kind, page_size=P, value_group=Gv, device=dev)
    pt = torch.from_numpy(pt_np).to(dev)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    flush_buf = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)

    def step():
        kvc.append(cache, K, V, start, pt)

    if args.profile_steps:
        for _ in range(args.profile_steps):
            flush_buf.sum()
            step()
        torch.cuda.synchronize()
        log("[bench] profile steps done")
        return
    for _ in range(args.warmup):
        flush_buf.sum()
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush_buf.sum()
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms = statistics.mean(step_ms)
    th = n_new * Ha
    value = th / (ms / 1e3)
    key_bytes, vb = 20, value_bytes(Gv)
    alg = th * (2 * D * 2 + key_bytes + vb)
    ach = alg / (ms / 1e3) / 1e9
    kern = "k_append_hadamard" if kind != "dense" else "k_append_mfma"
    log(f"[bench] append {ms * 1e3:.1f} us (median {statistics.median(step_ms) * 1e3:.1f}); {value:.3e} "
        f"token-heads/s; {ach:.0f} GB/s algorithmic = {100 * ach / HBM_PEAK_GBS:.1f}% of peak")
    result = {
        "metric": APPEND_METRIC, "value": value, "unit": "token-heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 in, f32 arithmetic, u8/u32 records out", "data": "synthetic",
        "config": {"workload": name, "new_tokens": n_new, "kv_heads": Ha, "head_dim": D, "value_group": Gv,
                   "page_size": P, "rotation": wl.rot, "kv_dtype": wl.kv_dtype,
                   "cache_flushed_between_steps": not args.no_flush},
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(kern, name),
                     "algorithmic_bytes_per_launch": alg, "avg_launch_us": round(ms * 1e3, 2)},
        "step_us_median": round(statistics.median(step_ms) * 1e3, 2),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"] = cpu_append_baseline(args, wl, K, V, cache, pt_np, rot)
    print(json.dumps(result), flush=True)


def cpu_append_baseline(args, wl, K, V, cache, pt_np, signs):
    """The oracle's key and value encode, untuned, on a bounded sample of the same append:
    the first tokens of every KV head, split over the host cores by (head, token block)."""
    import numpy as np

    import oracle

    D, P, Gv = wl.D, wl.P, wl.Gv
    Ha = K.shape[2]
    cores = len(os.sched_getaffinity(0))
    n = 2048  # tokens per head in the sample
    orot = (oracle.Rotation(oracle.ROT_HADAMARD, D, signs=signs) if wl.rot == "hadamard"
            else oracle.Rotation(oracle.ROT_DENSE, D, R16=signs))
    k = K[0, :n].float().cpu().numpy()
    v = V[0, :n].float().cpu().numpy()
    units = [(h, t0) for h in range(Ha) for t0 in range(0, n, 256)]

    def enc(u):
        h, t0 = u
        bits, nc = oracle.key_encode(orot, k[t0:t0 + 256, h])
        codes, sz = oracle.value_encode(v[t0:t0 + 256, h], D, Gv)
        return bits, nc, codes, sz

    reps = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        while True:
            res = list(ex.map(enc, units))
            reps += 1
            el = time.perf_counter() - t0
            if el * (reps + 1) / reps > args.cpu_seconds or reps >= 200:
                break
    cpu_value = reps * n * Ha / el
    # parity of the sample against the bytes the library wrote
    kb = cache.key_bits.cpu().numpy().view(np.uint32)
    kn = cache.key_nc.cpu().numpy().view(np.uint32)
    vc = cache.val_codes.cpu().numpy()
    vs = cache.val_sz.cpu().numpy().view(np.uint32)
    bad = 0
    for (h, t0_), (bits, nc, codes, sz) in zip(units, res):
        t = np.arange(t0_, t0_ + 256)
        pg, sl = pt_np[0, t // P], t % P
        ok = (np.array_equal(kb[pg, h, sl], bits) and np.array_equal(kn[pg, h, sl] & 0xFFFF, nc[:, 0])
              and np.all(np.abs((kn[pg, h, sl] >> 16).astype(np.int64) - nc[:, 1].astype(np.int64)) <= 1)
              and np.array_equal(vc[pg, h, sl], codes)
              and np.array_equal(vs[pg, h, sl], sz[..., 0].astype(np.uint32) | (sz[..., 1].astype(np.uint32) << 16)))
        bad += 0 if ok else 1
    log(f"[cpu] oracle append {cpu_value:.3e} token-heads/s on {cores} threads; sample units differing: {bad}")
    base = {"value": cpu_value, "unit": "token-heads/s", "cores": min(cores, len(units)), "kind": "oracle",
            "sample": f"first {n} tokens of each of {Ha} KV heads x {reps} repetition(s): the oracle's key and "
                      f"value encode in {len(units)} (head, 256-token) units", "seconds": round(el, 2)}
    return base, {"units": len(units), "units_differing": bad,
                  "bar": "sign bits, norms, codes, scale/zero bit-exact; correction within one binary16 ulp"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * 2**20 // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB five times")
        return

    if args.lazy:
        return run_lazy(args)
    if args.append:
        return run_append(args)

    import bit_kv_cache_compress_amd as kvc
    import workloads as W

    wl = workload(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    D, Hq, Hkv, B, P, Gv = wl.D, wl.Hq, wl.Hkv, wl.B, wl.P, wl.Gv
    lens = W.draw_seq_lens(wl)
    Lmax = int(lens.max())
    log(f"[bench] workload {wl.name}: B={B} Hq={Hq} Hkv={Hkv} L<={Lmax} top_p={wl.top_p} rot={wl.rot}")

    t0 = time.time()
    K, V, q = W.draw_device(wl, dev, L=Lmax)
    pt_np, npages = W.page_layout(wl, lens)
    kind, rot = W.draw_rotation(wl)
    center = None
    if args.center_keys:
        center = torch.zeros((Hkv, D), dtype=torch.float64, device=dev)
        for b in range(B):
            center += K[b, :int(lens[b]) - 1].double().sum(dim=0)
        center = (center / float(max(int(lens.sum()) - B, 1))).float()
    cache = kvc.KVCache(npages, Hkv, rot, rot_kind=kind, page_size=P, value_group=Gv, device=dev,
                        exact_keys=args.exact_keys, key_center=center, sketch_dim=args.sketch_dim)
    dither = None
    if args.stochastic_query:
        gd = torch.Generator(device=dev)
        gd.manual_seed(wl.seed(77))
        dither = torch.rand((B, Hq, D), generator=gd, device=dev, dtype=torch.float32)
    pt = torch.from_numpy(pt_np).to(dev)
    seq = torch.from_numpy(lens.astype(np.int32)).to(dev)
    # prefill tokens 0 .. len-2 of every sequence
    if np.all(lens == Lmax):
        kvc.append(cache, K[:, :Lmax - 1].contiguous(), V[:, :Lmax - 1].contiguous(),
                   torch.zeros(B, dtype=torch.int32, device=dev), pt)
    else:
        for b in range(B):
            n = int(lens[b]) - 1
            if n > 0:
                kvc.append(cache, K[b:b + 1, :n].contiguous(), V[b:b + 1, :n].contiguous(),
                           torch.zeros(1, dtype=torch.int32, device=dev), pt[b:b + 1].contiguous())
    idx_last = torch.from_numpy(lens.astype(np.int64) - 1).to(dev)
    ar = torch.arange(B, device=dev)
    k_new = K[ar, idx_last].unsqueeze(1).contiguous()  # [B, 1, Hkv, D]
    v_new = V[ar, idx_last].unsqueeze(1).contiguous()
    start = (seq - 1).contiguous()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kvc.decode_workspace_bytes(B, Hq, Hkv, Lmax, wl.top_p), dtype=torch.uint8, device=dev)
    # read-only sweep of 512 MiB between steps: evicts L2 and the 256 MB Infinity Cache
    # without leaving dirty lines behind (whose write-back would be charged to the next step).
    # A float32 buffer is summed in its own dtype, with no widening copy.
    flush_buf = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)

    def flush():
        flush_buf.sum()
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.1f}s, cache {cache.nbytes() / 2**20:.0f} MiB, "
        f"workspace {ws.numel() / 2**20:.1f} MiB")

    def step(dbg=None):
        if args.separate_append:
            kvc.append(cache, k_new, v_new, start, pt)
            kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=Lmax, out=out, workspace=ws,
                              debug_struct=dbg, q_dither=dither)
        else:  # the new tokens' encoding rides in the decode's first launch
            kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=Lmax, out=out, workspace=ws,
                              debug_struct=dbg, q_dither=dither, append=(k_new, v_new, start))

    if args.profile_steps:
        for _ in range(args.profile_steps):
            if not args.no_flush:
                flush()
            step()
        torch.cuda.synchronize()
        log("[bench] profile steps done")
        return

    for _ in range(args.warmup):
        if not args.no_flush:
            flush()
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # the step allocates nothing and synchronizes nowhere, so it can be captured as it is
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(args.warmup):
            if not args.no_flush:
                flush()
            run()
        torch.cuda.synchronize()

    # ---- timed region: K steps, per-step HIP events (flush outside the events)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush()
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    ms = statistics.mean(step_ms)
    tokens_heads = int(lens.astype(np.int64).sum()) * Hkv
    value = tokens_heads / (ms / 1e3)
    log(f"[bench] step {ms * 1e3:.1f} us (median {statistics.median(step_ms) * 1e3:.1f}, "
        f"p10 {np.percentile(step_ms, 10) * 1e3:.1f}, p90 {np.percentile(step_ms, 90) * 1e3:.1f}); "
        f"{value:.3e} KV token-heads/s")

    # ---- second timed region with per-stage events recorded by the library
    timers = [kvc.StageTimer() for _ in range(args.steps)]
    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        if not args.no_flush:
            flush()
        aev[i][0].record()
        if args.separate_append:
            kvc.append(cache, k_new, v_new, start, pt)
        aev[i][1].record()
        kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=Lmax, out=out, workspace=ws,
                          debug_struct=timers[i].struct(), q_dither=dither,
                          append=None if args.separate_append else (k_new, v_new, start))
    torch.cuda.synchronize()
    stage_ms = {}
    ran = ("query", "score", "hist", "attend", "merge") if wl.top_p < 1.0 else ("query", "attend", "merge")
    for t in timers:
        for k, v in t.elapsed_ms(ran).items():
            stage_ms.setdefault(k, []).append(v)
    stage_ms = {k: statistics.mean(v) for k, v in stage_ms.items()}
    if args.separate_append:
        stage_ms["append"] = statistics.mean(a.elapsed_time(b) for a, b in aev)
    log("[bench] stages (us): " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in stage_ms.items()))

    # ---- selection statistics (one untimed debug decode)
    sel_union = sel_entries = None
    masked_tokens = masked_entries = 0
    if wl.top_p < 1.0:
        dbg = kvc.DecodeDebug.allocate(B, Hq, Lmax, True, dev, scores=False)
        kvc.decode_attend(cache, q, seq, pt, top_p=wl.top_p, max_seq_len=Lmax, debug=dbg, q_dither=dither)
        torch.cuda.synchronize()
        G = Hq // Hkv
        mask = torch.zeros((B, Hkv, Lmax), dtype=torch.bool, device=dev)
        cnt = dbg.sel_count
        for h in range(Hq):
            idx = dbg.sel_idx[:, h].clamp(min=0).long()
            valid = torch.arange(Lmax, device=dev)[None, :] < cnt[:, h:h + 1]
            m = torch.zeros((B, Lmax), dtype=torch.bool, device=dev)
            m.scatter_(1, idx * valid, valid)
            mask[:, h // G] |= m
        sel_union = int(mask.sum())
        sel_entries = int(cnt.sum())
        # groups that the attention pass reads whole (the masked matrix-core chunk pass, which
        # reads no distances): every head dense (more than 64 kept per 2048 tokens), groups of 4
        # heads over pages of >= 64 tokens, each head keeping more than a quarter of its sequence
        L_b = seq.long()[:, None]
        masked_tokens = 0
        masked_entries = 0
        if G == 4 and P >= 64 and not args.exact_keys and bool((cnt.long() * 2048 > 64 * L_b).all()):
            grp = (cnt.long() * 4 > L_b).view(B, Hkv, G).all(dim=2)
            masked_tokens = int((grp.long() * L_b).sum())
            masked_entries = int((cnt.long().view(B, Hkv, G).sum(dim=2) * grp.long()).sum())
        if masked_tokens:
            log(f"[bench] the masked chunk pass reads {masked_tokens} token-KV-heads whole")
        sel_frac = float(cnt.sum()) / float(tokens_heads * G)
        log(f"[bench] Top-p kept {sel_frac * 100:.2f}% of (token, query head) pairs; "
            f"union over GQA groups {sel_union} token-KV-heads")
        del dbg, mask

    # ---- roofline of the dominant kernel (the stage with the longest average duration)
    G = Hq // Hkv
    kv_in = 2 if wl.kv_dtype == "f16" else 4
    key_bytes = 4 * (args.sketch_dim // 32 + 1)  # the key record: sign words and the norm/corr word
    topp = wl.top_p < 1.0
    exact = args.exact_keys and topp
    vb = value_bytes(Gv)
    new_tokens = B * Hkv  # the step appends one token per sequence and KV head
    append_alg = (2 * D * kv_in + key_bytes + vb + (2 * D if args.exact_keys else 0)) * new_tokens
    # algorithmic bytes per launch: every key record once (score pass; the full-softmax
    # attention pass reads keys itself), the value record of every attended token-KV-head once
    # (Top-p: the union over the KV head's query heads; with binary16 keys, also those keys)
    alg = {
        "score": key_bytes * tokens_heads,
        "attend": (vb + (2 * D if exact else 0)) * sel_union if topp else (key_bytes + vb) * tokens_heads,
        "hist": 0, "query": 0, "merge": 0, "append": append_alg}
    # what the design moves on top: 16-bit bin distances (written once, read by the histogram
    # and the attention pass), the kept tokens' key records re-read for their scores, and one
    # value record per kept (token, query head) rather than per KV head
    design = {
        "score": (key_bytes + DIST_BYTES * G) * tokens_heads if topp else key_bytes * tokens_heads,
        "attend": (DIST_BYTES * G * (tokens_heads - masked_tokens)
                   + ((2 * D if exact else key_bytes) + vb) * (sel_entries - masked_entries)
                   + (key_bytes + vb) * masked_tokens)
        if topp else (key_bytes + vb) * tokens_heads,
        "hist": DIST_BYTES * G * tokens_heads, "query": 0, "merge": 0, "append": append_alg}
    score_kernel = ("k_score_topp_mf" if G >= 4 else "k_score_topp") if topp else "k_score"
    # full softmax: the matrix-core kernel unless its A operand would fill fewer than 4 rows
    full_kernel = "k_attend_full_mf" if G * (D // Gv) >= 4 else "k_attend_full"
    kernel_names = {"score": score_kernel, "append": "k_append",
                    "attend": "k_attend_topp" if topp else full_kernel, "hist": "k_hist",
                    "query": "k_qprep", "merge": "k_merge"}
    dominant = max((k for k in stage_ms if k in alg), key=lambda k: stage_ms[k])
    t_dom = stage_ms[dominant] / 1e3
    ach = alg[dominant] / t_dom / 1e9
    variant = args.exact_keys or args.center_keys or args.stochastic_query or args.sketch_dim != D
    roofline = {"bound": "hbm", "kernel": kernel_names[dominant], "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": None if variant else measured_traffic(kernel_names[dominant], wl.name),
                "algorithmic_bytes_per_launch": alg[dominant],
                "avg_launch_us": round(stage_ms[dominant] * 1e3, 2),
                "design_bytes_per_launch": design[dominant],
                "design_frac": round(design[dominant] / t_dom / 1e9 / HBM_PEAK_GBS, 4)}
    # whole step, algorithmic minimum: every key once, the attended values once per KV head,
    # the appended tokens, the queries and the outputs
    qo = 2 * B * Hq * D * 4
    if topp:
        step_alg = append_alg + key_bytes * tokens_heads + (vb + (2 * D if exact else 0)) * sel_union + qo
    else:
        step_alg = append_alg + (key_bytes + vb) * tokens_heads + qo
    log(f"[bench] dominant {dominant}: {ach:.0f} GB/s algorithmic = {100 * ach / HBM_PEAK_GBS:.1f}% of peak "
        f"({design[dominant] / t_dom / 1e9:.0f} GB/s counting the design's bytes); whole step "
        f"{100 * step_alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS:.1f}% of peak")
    stage_alg = {k: {"us": round(stage_ms[k] * 1e3, 2), "algorithmic_bytes": alg[k], "design_bytes": design[k],
                     "frac": round(alg[k] / (stage_ms[k] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
                 for k in stage_ms if k in alg}

    result = {
        "metric": METRIC, "value": value, "unit": "KV token-heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i32 (1-bit x int4 popcount) + f32", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": Lmax,
                   "head_dim": D, "top_p": wl.top_p, "value_group": Gv, "page_size": P, "rotation": wl.rot,
                   "kv_dtype": wl.kv_dtype,
                   "step": "append 1 token per sequence + decode attention"
                           + (" (two calls)" if args.separate_append else " (one call, fused append)"),
                   "cache_flushed_between_steps": not args.no_flush, "exact_keys": args.exact_keys,
                   "key_center": args.center_keys, "stochastic_query": args.stochastic_query,
                   "sketch_dim": args.sketch_dim, "hip_graph": args.graph},
        "roofline": roofline,
        "step_hbm_frac_algorithmic": round(step_alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": step_alg,
        "query_head_tokens_per_s": value * (Hq // Hkv),
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "stages": stage_alg,
        "step_us_median": round(statistics.median(step_ms) * 1e3, 2),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 3),
    }
    if sel_union is not None:
        result["topp_selected_union_token_kv_heads"] = sel_union
        result["topp_selected_token_query_heads"] = sel_entries

    if variant and not args.no_cpu_baseline:
        log("[cpu] no oracle baseline for the variant modes (the default run has it)")
    elif not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(args, wl, K, V, q, lens, pt_np, kind, rot,
                                                                      out, value)
    print(json.dumps(result), flush=True)


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this kernel and
    workload, when the kernel source is unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        srcs = rec["source"] if isinstance(rec["source"], list) else [rec["source"]]
        h = hashlib.sha256()
        for f in srcs:  # the kernel's file and the headers listed with it, in order
            h.update(open(os.path.join(ROOT, "bit_kv_cache_compress_amd", "csrc", f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


def cpu_baseline(args, wl, K, V, q, lens, pt_np, kind, rot, gpu_out, gpu_value):
    """The oracle, untuned, on a bounded sample of the same workload: the decode step of a
    few whole (sequence, KV head) units -- its G query heads over every cached token --
    run on the host cores, one unit per thread."""
    import numpy as np

    import oracle

    G = wl.Hq // wl.Hkv
    cores = len(os.sched_getaffinity(0))
    units = [(b, h) for b in range(wl.B) for h in range(wl.Hkv)][:max(1, min(wl.B * wl.Hkv, cores))]
    orot = oracle.Rotation(oracle.ROT_DENSE if kind == "dense" else oracle.ROT_HADAMARD, wl.D,
                           R16=rot if kind == "dense" else None, signs=rot if kind != "dense" else None)
    log(f"[cpu] encoding {len(units)} units with the oracle on {cores} cores")
    t0 = time.time()

    def encode(u):
        b, h = u
        n = int(lens[b])
        k = K[b, :n, h].float().cpu().numpy()
        v = V[b, :n, h].float().cpu().numpy()
        bits, nc = oracle.key_encode(orot, k)
        codes, sz = oracle.value_encode(v, wl.D, wl.Gv)
        return bits, nc, codes, sz

    with ThreadPoolExecutor(cores) as ex:
        enc = list(ex.map(encode, units))
    log(f"[cpu] oracle caches built in {time.time() - t0:.1f}s")
    qn = q.cpu().numpy()

    def decode_unit(i):
        b, h = units[i]
        bits, nc, codes, sz = enc[i]
        outs = []
        for hh in range(h * G, (h + 1) * G):
            qe = oracle.query_encode(orot, qn[b, hh][None, :])
            _, _, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], wl.D)
            if wl.top_p < 1.0:
                sel = oracle.topp(s, wl.top_p, wl.D)["idx"]
                outs.append(oracle.attend(s, codes, sz, wl.D, wl.Gv, sel))
            else:
                outs.append(oracle.attend(s, codes, sz, wl.D, wl.Gv))
        return outs

    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        while True:
            res = list(ex.map(decode_unit, range(len(units))))
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed * (reps + 1) / reps > args.cpu_seconds or reps >= 50:
                break
    work = reps * sum(int(lens[b]) for b, _ in units)
    cpu_value = work / elapsed
    # parity of the same sample against the GPU step's output
    go = gpu_out.cpu().numpy()
    worst = 0.0
    for (b, h), outs in zip(units, res):
        for j, hh in enumerate(range(h * G, (h + 1) * G)):
            ref = outs[j]
            worst = max(worst, float(np.abs(go[b, hh] - ref).max() / np.abs(ref).max()))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    log(f"[cpu] oracle {cpu_value:.3e} KV token-heads/s on {cores} threads ({model}); "
        f"GPU/CPU {gpu_value / cpu_value:.0f}x; sample max rel err {worst:.2e}")
    base = {"value": cpu_value, "unit": "KV token-heads/s", "cores": min(cores, len(units)), "kind": "oracle",
            "sample": f"{len(units)} (sequence, KV head) units x {reps} repetition(s): query encode, proxy "
                      f"scores, Top-p and attention of their {G} query heads over {int(lens[units[0][0]])} "
                      f"tokens (cache encoded untimed)", "cpu_model": model, "seconds": round(elapsed, 2)}
    return base, {"units": len(units), "max_rel_err_vs_oracle": worst, "tolerance": 2e-3}


if __name__ == "__main__":
    main()
