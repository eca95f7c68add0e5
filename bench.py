"""Benchmark: fused LUT decode attention from 4-bit Hadamard/Lloyd-Max key codes.

One step = one decode step of the whole hot path on one GPU, one launch of
kvq_decode_attn_append:
  1. write path: encode the new token's key of every (batch, kv head) into the
     code cache (norm + packed codes) at position T-1;
  2. read path: rotate the queries, build the per-head LUTs in LDS, score all
     T cached keys (the new one included) from their codes, online softmax, AV
     product over fp16 V, split merge -> attention output [B][Hq][d].

Workload (default): B=8, Hq=32, Hkv=4, d=64, b=4, T=32768 (1.1B-Llama-like
long-context decode), seeded synthetic inputs.  R >= 4 copies of the cache at
distinct addresses are rotated so every step streams from HBM rather than the
256 MB last-level cache.

Prints ONE JSON line on stdout (human-readable detail on stderr).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "keys scored/sec and % of HBM roofline, fused 4-bit LUT decode attn, B=8 T=32k"
HBM_PEAK_GBS = 8000.0
# Measured HBM traffic of the decode-attention kernel on this workload (rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, scaled by a plain copy of known size).  It is reported only while the library sources hash to
# the digest recorded with the counters; after any change to them the figure is stale and traffic is null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_longctx_hbm_traffic.txt")
TRAFFIC_FILE_QV = os.path.join(ROOT, "profiles", "qv_decode_kernel_longctx_hbm_traffic.txt")
TRAFFIC_FILE_ENC = os.path.join(ROOT, "profiles", "hlm_encode_kernel_sweep_b4_B64_hbm_traffic.txt")


def library_source_digest():
    """sha256 over the HIP/C++ sources and headers of libkvq (names and contents, sorted by name)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_encode_amd", "csrc")
    files = sorted(f for f in os.listdir(csrc) if f.endswith((".h", ".hip", ".cpp")))
    for f in files + ["kvq.h"]:
        path = os.path.join(ROOT, "include", f) if f == "kvq.h" else os.path.join(csrc, f)
        h.update(f.encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch from the committed counter summary, or None if absent or stale."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != library_source_digest() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def settle(torch, replay, seconds, min_replays=3, max_replays=2000):
    """Untimed replays of the timed graph until the GPU has run this load for `seconds` of wall time (at least
    `min_replays`).  The GPU's clocks reach their steady state under a sustained load only after about a
    second: the long-context step measured 39.4 us after 24 ms of such replays and 36.9 us after 0.8 s."""
    t0 = time.perf_counter()
    n = 0
    while n < min_replays or (time.perf_counter() - t0 < seconds and n < max_replays):
        replay()
        torch.cuda.synchronize()
        n += 1
    return n


def copy_calibration(torch):
    """A plain device-to-device copy of known size (256 MiB read + 256 MiB written per launch, three launches):
    the kernel whose FETCH_SIZE / WRITE_SIZE readings scale the counters of the library's kernels."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def pmc_summary(path, kernel_regex):
    """Per-dispatch means of the counters in a rocprofv3 --pmc CSV (a file, or a directory searched for
    *counter_collection.csv), for the dispatches whose kernel name matches kernel_regex, grouped by kernel
    and grid size; the plain copy kernel is listed too, for scaling FETCH_SIZE / WRITE_SIZE."""
    import csv
    import glob

    files = [path] if os.path.isfile(path) else sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                                                recursive=True))
    if not files:
        print("no *counter_collection.csv under %s" % path)
        return 1
    pat = re.compile(kernel_regex)
    groups = {}  # (short name, grid) -> counter -> [values]
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if not (pat.search(name) or "copyBuffer" in name):
                    continue
                short = name.split("(")[0].replace("void ", "")[:90]
                key = (short, r.get("Grid_Size", "?"), r.get("Workgroup_Size", "?"))
                d = groups.setdefault(key, {})
                d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for (short, grid, wg), counters in sorted(groups.items()):
        n = max(len(v) for v in counters.values())
        print("%s  grid=%s wg=%s  dispatches=%d" % (short, grid, wg, n))
        for cn in sorted(counters):
            v = counters[cn]
            print("  %-28s mean %14.1f  min %14.1f  max %14.1f" % (cn, sum(v) / len(v), min(v), max(v)))
    return 0


def algorithmic_bytes(shape, bpk, append=False):
    """Bytes a decode step must move: codes + fp32 norms + V of every cached key, and q (outputs not
    credited); with append, also the new keys read and their codes and norms written."""
    keys = shape.B * shape.Hkv * shape.T
    vb = 2 if shape.dtype == "f16" else 4
    n = keys * (bpk + 4 + shape.d * vb) + shape.B * shape.Hq * shape.d * vb
    if append:
        n += shape.B * shape.Hkv * (shape.d * vb + bpk + 4)
    return n


def oracle_threads():
    """Host threads for the oracle: the cores this process may run on, at most 16 (one GPU's share of a box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def time_oracle(tasks, min_seconds, threads):
    """Wall time of passes over `tasks` (callables; the oracle's ctypes calls release the GIL, so a thread pool
    runs them on `threads` cores), repeated until min_seconds have passed.  Returns (passes, seconds)."""
    from concurrent.futures import ThreadPoolExecutor

    passes, elapsed = 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while passes == 0 or elapsed < min_seconds:
            t0 = time.perf_counter()
            for _ in ex.map(lambda f: f(), tasks):
                pass
            elapsed += time.perf_counter() - t0
            passes += 1
    return passes, elapsed


def oracle_record(tasks, units_per_pass, unit, min_seconds, what):
    """The oracle timed on all of the host's cores (the reported figure) and on one thread (beside it)."""
    threads = oracle_threads()
    p1, s1 = time_oracle(tasks, min(3.0, min_seconds / 4), 1)
    pn, sn = time_oracle(tasks, min_seconds, threads)
    return {"value": pn * units_per_pass / sn, "unit": unit, "cores": threads, "kind": "oracle",
            "value_1thread": p1 * units_per_pass / s1,
            "sample": "%s: %d pass(es) in %.1f s on %d thread(s) (a thread pool over the tasks; %d pass(es) in "
                      "%.1f s on one thread for value_1thread)" % (what, pn, sn, threads, p1, s1)}


def cpu_baseline(shape, signs, q, min_seconds=5.0):
    """The fp64 oracle on the same decode step: for every (batch, kv head), the write path's encode of the new key
    and decode attention of that kv head's query heads over all T cached keys."""
    import numpy as np

    import oracle
    import workloads as W

    lv, th = oracle.codebook(shape.d, shape.b)
    scale = 1.0 / math.sqrt(shape.d)
    G = shape.Hq // shape.Hkv
    newk = W.new_keys(shape).astype(np.float64)
    q64 = q.astype(np.float64)
    tasks = []
    for bi in range(shape.B):  # the prefilled cache: encoded by the oracle itself, untimed
        keys = W.keys(shape, batches=[bi])
        codes, norms, _, _ = oracle.encode_keys(th, signs, keys, shape.b)
        v = W.values(shape, batches=[bi]).astype(np.float64)
        for h in range(shape.Hkv):
            args = (q64[bi:bi + 1, h * G:(h + 1) * G], codes[:, h:h + 1], norms[:, h:h + 1], v[:, h:h + 1],
                    newk[bi:bi + 1, h:h + 1])

            def task(a=args):
                oracle.encode_keys(th, signs, a[4], shape.b)                       # write path of the step
                oracle.decode_attn(lv, signs, a[0], a[1], a[2], a[3], scale)     # read path of the step
            tasks.append(task)
    return oracle_record(tasks, shape.B * shape.Hq * shape.T, "keys/s", min_seconds,
                         "the full decode step (B=%d, Hq=%d, T=%d): fp64 C oracle encode of the new keys + decode "
                         "attention, %d (batch, kv head) tasks" % (shape.B, shape.Hq, shape.T, len(tasks)))


def cpu_baseline_qv(shape, signs, q, min_seconds=5.0):
    """The fp64 oracle on the quantized-value decode step, per (batch, kv head)."""
    import numpy as np

    import oracle
    import workloads as W

    lv, th = oracle.codebook(shape.d, shape.b)
    scale = 1.0 / math.sqrt(shape.d)
    G = shape.Hq // shape.Hkv
    q64 = q.astype(np.float64)
    tasks = []
    for bi in range(shape.B):  # keys and values encoded by the oracle itself, untimed
        codes, norms, _, _ = oracle.encode_keys(th, signs, W.keys(shape, batches=[bi]), shape.b)
        vcodes, vnorms, _, _ = oracle.encode_keys(th, signs, W.values(shape, batches=[bi]), shape.b)
        for h in range(shape.Hkv):
            args = (q64[bi:bi + 1, h * G:(h + 1) * G], codes[:, h:h + 1], norms[:, h:h + 1], vcodes[:, h:h + 1],
                    vnorms[:, h:h + 1])

            def task(a=args):
                oracle.decode_attn_qv(lv, signs, a[0], a[1], a[2], a[3], a[4], scale)
            tasks.append(task)
    return oracle_record(tasks, shape.B * shape.Hq * shape.T, "keys/s", min_seconds,
                         "the full quantized-value decode step (B=%d, Hq=%d, T=%d): fp64 C oracle (value "
                         "dequantization + decode attention), %d (batch, kv head) tasks"
                         % (shape.B, shape.Hq, shape.T, len(tasks)))


def cpu_baseline_pot(shape, q, bits, mantissa, min_seconds=5.0):
    """The fp64 oracle on the power-of-two decode step, per (batch, kv head)."""
    import numpy as np

    import oracle
    import workloads as W

    scale = 1.0 / math.sqrt(shape.d)
    G = shape.Hq // shape.Hkv
    newk = W.new_keys(shape).astype(np.float64)
    q64 = q.astype(np.float64)
    tasks = []
    for bi in range(shape.B):  # the prefilled cache, encoded by the oracle itself, untimed
        codes, scales, _ = oracle.pot_encode(W.keys(shape, batches=[bi]), bits, mantissa)
        v = W.values(shape, batches=[bi]).astype(np.float64)
        for h in range(shape.Hkv):
            args = (q64[bi:bi + 1, h * G:(h + 1) * G], codes[:, h:h + 1], scales[:, h:h + 1], v[:, h:h + 1],
                    newk[bi:bi + 1, h:h + 1])

            def task(a=args):
                oracle.pot_encode(a[4], bits, mantissa)                                  # write path
                oracle.pot_decode_attn(a[0], a[1], a[2], a[3], bits, mantissa, scale)    # read path
            tasks.append(task)
    return oracle_record(tasks, shape.B * shape.Hq * shape.T, "keys/s", min_seconds,
                         "the full power-of-two decode step (B=%d, Hq=%d, T=%d): fp64 C oracle encode of the new "
                         "keys + decode attention, %d (batch, kv head) tasks" % (shape.B, shape.Hq, shape.T, len(tasks)))


def cpu_baseline_encode(shape, signs, min_seconds=5.0):
    """The fp64 oracle's encode on batch 0 of the workload, per kv head."""
    import oracle
    import workloads as W

    _, th = oracle.codebook(shape.d, shape.b)
    keys = W.keys(shape, batches=[0])
    tasks = []
    for h in range(shape.Hkv):
        kh = keys[:, h:h + 1].copy()

        def task(k=kh):
            oracle.encode_keys(th, signs, k, shape.b)
        tasks.append(task)
    n = keys.shape[0] * keys.shape[1] * keys.shape[2]
    return oracle_record(tasks, n, "keys/s", min_seconds,
                         "batch 0 of the workload (Hkv=%d x T=%d keys, d=%d): fp64 C oracle encode, %d kv-head tasks"
                         % (shape.Hkv, shape.T, shape.d, len(tasks)))


def run_encode(K, torch, a):
    """The write path at the batch-64 sweep shape (B=64, Hkv=8, T=8192, d=128, b=4, fp16 keys with
    per-(kv head, channel) LogNormal(0,1) scales): kvq_encode_keys over the whole cache, replayed from a HIP
    graph, with two key sources and four code/norm buffers in rotation."""
    import workloads as W

    dev = torch.device("cuda:0")
    shape = next(s for s in W.SWEEP if s.b == 4 and s.B == 64)
    B, Hkv, d, T, b = shape.B, shape.Hkv, shape.d, shape.T, shape.b
    eprint("generating %s: B=%d Hkv=%d d=%d b=%d T=%d" % (shape.name, B, Hkv, d, b, T))
    signs = W.signs(shape)
    cb = K.kvq_build_codebook(d, b)
    bpk = cb.bytes_per_key
    keys0 = torch.empty((B, Hkv, T, d), dtype=torch.float16, device=dev)
    for bi in range(B):  # the workload's seeded keys, one batch at a time
        keys0[bi] = torch.from_numpy(W.keys(shape, batches=[bi])[0]).to(dev)
    srcs = [keys0, keys0.clone()]
    outs = [(torch.empty((B, Hkv, T, bpk), dtype=torch.uint8, device=dev),
             torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)) for _ in range(4)]

    def step(i):
        c, n = outs[i % len(outs)]
        K.kvq_encode_keys(cb, signs, srcs[i % len(srcs)], c, n)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(a.warmup, len(outs))):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(a.steps):
            step(i)
    settle(torch, g.replay, a.settle_seconds)
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    t_start.record()
    g.replay()
    t_stop.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / a.steps
    if a.calibrate_copy:
        copy_calibration(torch)
    n_keys = B * Hkv * T
    value = n_keys / (ms_per_step * 1e-3)
    alg_bytes = n_keys * (2 * d + bpk + 4)
    achieved = alg_bytes / (ms_per_step * 1e-3) / 1e9
    eprint("encode %.4f ms -> %.4g keys/s; %d algorithmic bytes -> %.1f GB/s = %.1f%% of %.0f GB/s" %
           (ms_per_step, value, alg_bytes, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))
    cpu = None
    if not a.no_cpu_baseline:
        eprint("timing the CPU oracle on a bounded sample (~%.0f s)" % a.cpu_seconds)
        cpu = cpu_baseline_encode(shape, signs, a.cpu_seconds)
        eprint("cpu oracle: %.4g keys/s (%s)" % (cpu["value"], cpu["sample"]))
    rec = {
        "metric": "cached keys encoded/sec and % of HBM roofline, Hadamard/Lloyd-Max write path, B=64 T=8k",
        "value": value, "unit": "keys/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 (norm, rotation, code search on fp16 keys)", "data": "synthetic",
        "config": {"workload": "sweep encode: B=64 Hkv=8 d=128 b=4 T=8192, fp16 keys", "B": B, "Hkv": Hkv, "d": d,
                   "b": b, "T": T, "k_dtype": "f16",
                   "step": "one kvq_encode_keys call: norm, rotation, codes and norms of B*Hkv*T keys",
                   "key_sources_rotated": len(srcs), "outputs_rotated": len(outs)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(TRAFFIC_FILE_ENC),
                     "kernel": "hlm_encode_kernel (norm + in-register Walsh-Hadamard transform + cell-table "
                               "code search + packing)",
                     "avg_launch_ms": ms_per_step, "algorithmic_bytes": alg_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_stream(K, torch, a):
    """The streaming ceiling of the long-context decode step: kvq_stream_read reads the same codes, norms and fp16
    V (171,966,464 bytes) with the decode kernel's grid, split and access pattern and does nothing else; four
    copies of the cache rotate, as in the decode step's timing."""
    import workloads as W

    dev = torch.device("cuda:0")
    shape = W.LONGCTX
    B, Hq, Hkv, d, T, b = shape.B, shape.Hq, shape.Hkv, shape.d, shape.T, shape.b
    bpk = d * b // 8
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    caches = []
    for _ in range(a.caches):  # contents do not matter to a plain read; random bytes of the right sizes
        caches.append((torch.randint(0, 256, (B, Hkv, T, bpk), dtype=torch.uint8, device=dev, generator=g),
                       torch.rand((B, Hkv, T), device=dev, generator=g),
                       torch.randn((B, Hkv, T, d), device=dev, generator=g).half()))
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cb = K.kvq_build_codebook(d, b)
    ws = K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, a.splits)
    splits = ws // (B * Hq * (d + 4) * 4) if ws else 1  # the decode step's split count

    def step(i):
        c, n, v = caches[i % len(caches)]
        K.kvq_stream_read(c, n, v, splits, sink)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(a.warmup, len(caches))):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for i in range(a.steps):
            step(i)
    settle(torch, gr.replay, a.settle_seconds)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    gr.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps
    nbytes = B * Hkv * T * (bpk + 4 + 2 * d)
    gbs = nbytes / (ms * 1e-3) / 1e9
    eprint("plain read %.4f ms: %d bytes -> %.1f GB/s = %.1f%% of %.0f GB/s" % (ms, nbytes, gbs,
                                                                             100 * gbs / HBM_PEAK_GBS, HBM_PEAK_GBS))
    rec = {
        "metric": "streaming ceiling: plain read of the long-context decode cache with the decode access pattern, "
                  "GB/s and % of HBM roofline",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32 (checksum only)",
        "data": "synthetic",
        "config": {"workload": "longctx cache: B=8 Hkv=4 d=64 b=4 T=32768, codes + fp32 norms + fp16 V",
                   "B": B, "Hkv": Hkv, "d": d, "b": b, "T": T, "t_splits": int(splits),
                   "caches_rotated": len(caches),
                   "step": "one kvq_stream_read launch: 12-wave workgroups, 64 tokens per wave and chunk, one chunk "
                           "ahead, non-temporal loads"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "stream_read_kernel",
                     "avg_launch_ms": ms, "algorithmic_bytes": nbytes},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_suite(K, torch, reps=5, calls=30, only=None, settle_seconds=0.3):
    """Every configuration of the method on one GPU: read path (fused decode, scores alone), write path
    (encode), and the PQ variant.  Inputs are drawn on the GPU from a seeded generator with the workloads'
    shapes and distributions (normal keys and values; per-(kv head, channel) LogNormal(0,1) scales for the
    Llama-8B-like shapes, per-token LogNormal(0,0.5) key scales for the long-context one); at least four
    distinct caches rotate so every call streams from HBM.  Each figure is the median over `reps` graph
    replays of `calls` calls.  Prints one table row per (workload, operation)."""
    import workloads as W

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    rows = []

    def rnd(*shape):
        return torch.randn(shape, device=dev, dtype=torch.float32, generator=gen)

    def draw_keys(sh, T):
        k = rnd(sh.B, sh.Hkv, T, sh.d)
        if sh.key_scale == "channel_lognormal":
            k *= torch.exp(rnd(1, sh.Hkv, 1, sh.d))
        elif sh.key_scale == "token_lognormal":
            k *= torch.exp(0.5 * rnd(sh.B, sh.Hkv, T, 1))
        return k.half()

    def draw_values(sh, T):
        v = rnd(sh.B, sh.Hkv, T, sh.d)
        if sh.v_scale == "channel_lognormal":
            v *= torch.exp(rnd(1, sh.Hkv, 1, sh.d))
        return v.half()

    def timed(fn, n_rot):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(max(n_rot, 3)):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                fn(i)
        # untimed replays until the clocks have settled under this load (a few replays alone left the short
        # kernels 1-5 us per call slower than their steady state)
        settle(torch, g.replay, settle_seconds)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / calls)
        ts.sort()
        return ts[len(ts) // 2] * 1e-3  # seconds per call

    ops = ("decode", "append+dec", "score", "encode", "decode-qv", "pot-decode", "pot-encode", "pot-m-decode",
           "pot-m-encode", "select/cand")

    def want(name, op=None):
        """--only: a regular expression searched in "<workload> <operation>"; rows that do not match are skipped."""
        if only is None:
            return True
        return any(re.search(only, name + " " + o) for o in ((op,) if op else ops))

    def measure(name, op, fn, n_rot, nbytes, keys_scored, cached):
        if want(name, op):
            row(name, op, timed(fn, n_rot), nbytes, keys_scored, cached)

    def row(name, op, sec, nbytes, keys_scored, cached):
        rows.append((name, op, sec * 1e6, nbytes / sec / 1e9, 100 * nbytes / sec / 1e9 / HBM_PEAK_GBS,
                     keys_scored / sec if keys_scored else 0.0, cached / sec))
        eprint("%-22s %-10s %10.2f us %9.1f GB/s %6.1f%%  %10.3g keys-scored/s %10.3g cached-keys/s" % rows[-1])

    hlm = [("llama8b", W.LLAMA8B), ("longctx", W.LONGCTX)] + [(s.name, s) for s in W.SWEEP]
    for name, sh in hlm:
        if not want(name):
            continue
        B, Hq, Hkv, d, T, b = sh.B, sh.Hq, sh.Hkv, sh.d, sh.T, sh.b
        cb = K.kvq_build_codebook(d, b)
        bpk = cb.bytes_per_key
        signs = W.signs(sh)
        per_cache = B * Hkv * T * (bpk + 4 + 2 * d)
        n_rot = max(4, int(math.ceil(1.2e9 / per_cache)))  # >= 4 caches and >= 1.2 GB in rotation
        caches = []
        keys = None
        for r in range(n_rot):
            if r == 0:
                keys = draw_keys(sh, T)
                codes = torch.empty((B, Hkv, T, bpk), dtype=torch.uint8, device=dev)
                norms = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
                K.kvq_encode_keys(cb, signs, keys, codes, norms)
                caches.append((codes, norms, draw_values(sh, T)))
            else:
                c0, n0, v0 = caches[0]
                caches.append((c0.clone(), n0.clone(), v0.clone()))
        q = rnd(B, Hq, d).half()
        out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
        ws = torch.zeros(max(K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, 0), 16), dtype=torch.uint8, device=dev)
        nk = draw_keys(sh, 1)[:, :, 0, :].contiguous()

        def dec(i):
            c, n, v = caches[i % n_rot]
            K.kvq_decode_attn(cb, signs, q, c, n, v, out=out, workspace=ws)

        def app(i):
            c, n, v = caches[i % n_rot]
            K.kvq_decode_attn_append(cb, signs, nk, q, c, n, v, out=out, workspace=ws)

        scores = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)

        def score(i):
            c, n, _ = caches[i % n_rot]
            K.kvq_score(cb, signs, q, c, n, scores=scores)

        rd = algorithmic_bytes(sh, bpk)
        if want(name, "decode"):
            timed(dec, n_rot)  # untimed: the first graph of a workload runs slower (clocks, page tables)
        measure(name, "decode", dec, n_rot, rd, B * Hq * T, B * Hkv * T)
        measure(name, "append+dec", app, n_rot, algorithmic_bytes(sh, bpk, append=True), B * Hq * T, B * Hkv * T)
        measure(name, "score", score, n_rot, B * Hkv * T * (bpk + 4) + B * Hq * T * 4, B * Hq * T, B * Hkv * T)

        # the encode reads its keys from n_rot copies too, so that they stream from HBM rather than the
        # last-level cache
        key_srcs = [keys] + [keys.clone() for _ in range(n_rot - 1)]

        def enc(i):
            c, n, _ = caches[i % n_rot]
            K.kvq_encode_keys(cb, signs, key_srcs[i % n_rot], c, n)

        measure(name, "encode", enc, n_rot, B * Hkv * T * (2 * d + bpk + 4), 0, B * Hkv * T)

        # values stored with the same codec (rotated-domain AV, one inverse transform per head)
        vcs = []
        for r in range(n_rot):
            if r == 0:
                vc0 = torch.empty((B, Hkv, T, bpk), dtype=torch.uint8, device=dev)
                vn0 = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
                K.kvq_encode_keys(cb, signs, caches[0][2], vc0, vn0)
                vcs.append((vc0, vn0))
            else:
                vcs.append((vcs[0][0].clone(), vcs[0][1].clone()))

        def dec_qv(i):
            c, n, _ = caches[i % n_rot]
            vc, vn = vcs[i % n_rot]
            K.kvq_decode_attn_qv(cb, signs, q, c, n, vc, vn, out=out, workspace=ws)

        measure(name, "decode-qv", dec_qv, n_rot, B * Hkv * T * 2 * (bpk + 4) + B * Hq * d * 2, B * Hq * T,
            B * Hkv * T)
        del vcs

        # power-of-two key codes of the same width (shift-accumulate page), plain and with the mantissa term
        for mant in ((0, 1) if b >= 2 else ()):
            pcb = K.kvq_build_codebook_pot(d, b, mant)
            pcs = []
            for r in range(n_rot):
                if r == 0:
                    pc0 = torch.empty((B, Hkv, T, bpk), dtype=torch.uint8, device=dev)
                    ps0 = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
                    K.kvq_encode_keys(pcb, None, keys, pc0, ps0)
                    pcs.append((pc0, ps0))
                else:
                    pcs.append((pcs[0][0].clone(), pcs[0][1].clone()))

            def pot_dec(i):
                c, n = pcs[i % n_rot]
                K.kvq_decode_attn(pcb, None, q, c, n, caches[i % n_rot][2], out=out, workspace=ws)

            def pot_enc(i):
                c, n = pcs[i % n_rot]
                K.kvq_encode_keys(pcb, None, key_srcs[i % n_rot], c, n)

            tag = "pot-m" if mant else "pot"
            measure(name, tag + "-decode", pot_dec, n_rot, rd, B * Hq * T, B * Hkv * T)
            measure(name, tag + "-encode", pot_enc, n_rot, B * Hkv * T * (2 * d + bpk + 4), 0, B * Hkv * T)
            del pcs
        del caches, keys, key_srcs, scores
        torch.cuda.empty_cache()

    # product quantization (LOOKAT-style ADC) at the GPT-2-small-like shapes: byte codes (K = 256) and
    # 4-bit codes (K = 16, two subspaces per byte) at 32x and 64x compression
    for sh in (W.PQ_GPT2, W.PQ4_GPT2_32X, W.PQ4_GPT2_64X):
        if not want(sh.name):
            continue
        B, H, d, T, m, Kc = sh.B, sh.Hq, sh.d, sh.T, sh.m, sh.K
        cent = rnd(H, m, Kc, d // m)
        cb = K.kvq_codebook_pq(d, m, Kc, H, cent)
        bpk = cb.bytes_per_key
        n_rot = 8
        keys = rnd(B, H, T, d).half()
        codes0 = torch.empty((B, H, T, bpk), dtype=torch.uint8, device=dev)
        K.kvq_encode_keys(cb, None, keys, codes0)
        vals = rnd(B, H, T, d).half()
        caches = [(codes0, vals)] + [(codes0.clone(), vals.clone()) for _ in range(n_rot - 1)]
        q = rnd(B, H, d).half()
        out = torch.empty((B, H, d), dtype=torch.float16, device=dev)
        ws = torch.zeros(max(K.kvq_decode_attn_workspace(cb, B, H, H, T, 0), 16), dtype=torch.uint8, device=dev)
        scores = torch.empty((B, H, T), dtype=torch.float32, device=dev)

        def pq_dec(i):
            c, v = caches[i % n_rot]
            K.kvq_decode_attn(cb, None, q, c, None, v, out=out, workspace=ws)

        def pq_score(i):
            c, _ = caches[i % n_rot]
            K.kvq_score(cb, None, q, c, None, scores=scores)

        def pq_enc(i):
            c, _ = caches[i % n_rot]
            K.kvq_encode_keys(cb, None, keys, c)

        nkeys = B * H * T
        measure(sh.name, "decode", pq_dec, n_rot, nkeys * (bpk + 2 * d) + B * H * d * 2, nkeys, nkeys)
        measure(sh.name, "score", pq_score, n_rot, nkeys * (bpk + 4), nkeys, nkeys)
        measure(sh.name, "encode", pq_enc, n_rot, nkeys * (2 * d + bpk), 0, nkeys)
        del caches, keys, vals
    torch.cuda.empty_cache()
    if not want("signsel_200"):
        return rows

    # one-time sign-pattern selection: 200 candidates on 8 calibration samples of 512 keys.  The call is
    # synchronous (it returns the ranking to the host), so it is timed by wall clock, not in a graph; the
    # row reports the time per candidate (an encode and a decode of the calibration keys plus the error).
    sh = W.SIGNSEL
    B, Hq, Hkv, d, T, b = sh.B, sh.Hq, sh.Hkv, sh.d, sh.T, sh.b
    cb = K.kvq_build_codebook(d, b)
    cands = W.sign_candidates(sh)
    C = cands.shape[0]
    q, keys, vals = rnd(B, Hq, d).half(), draw_keys(sh, T), draw_values(sh, T)
    ws = torch.empty(K.kvq_select_signs_workspace(cb, B, Hq, Hkv, T, C), dtype=torch.uint8, device=dev)
    K.kvq_select_signs(cb, cands, q, keys, vals, workspace=ws)
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        K.kvq_select_signs(cb, cands, q, keys, vals, workspace=ws)
        ts.append(time.perf_counter() - t0)
    ts.sort()
    sel = ts[len(ts) // 2]
    nkeys = B * Hkv * T
    bpk = cb.bytes_per_key
    per_cand = nkeys * (2 * d + bpk + 4) + nkeys * (bpk + 4 + 2 * d) + 2 * B * Hq * d * 4
    row("signsel_200", "select/cand", sel / C, per_cand, B * Hq * T, nkeys)
    eprint("signsel_200: whole selection %.2f ms for %d candidates" % (sel * 1e3, C))
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed replays of the timed graph for this long before the timed one")
    ap.add_argument("--caches", type=int, default=4, help="distinct cache copies rotated across steps")
    ap.add_argument("--splits", type=int, default=0, help="T splits (0 = library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device copy (a known-size kernel for scaling HBM counters)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the headline step, time every workload and operation (table on stderr)")
    ap.add_argument("--only", default=None, metavar="REGEX",
                    help="with --suite: time only the rows whose \"<workload> <operation>\" matches REGEX "
                         "(e.g. 'longctx score')")
    ap.add_argument("--variant", choices=("append", "qv", "pot", "encode", "stream"), default="append",
                    help="append: the fused append + decode step over fp16 V (default); qv: decode attention "
                         "with the values stored as codes of the same codec (kvq_decode_attn_qv); pot: the fused "
                         "step with 4-bit power-of-two key codes (with the mantissa term) instead; encode: the "
                         "write path alone at the batch-64 sweep shape (kvq_encode_keys); stream: a plain read "
                         "of the long-context cache with the decode kernel's grid and access pattern "
                         "(kvq_stream_read), the streaming ceiling the decode step is measured against")
    ap.add_argument("--pmc-summary", default=None, metavar="PATH",
                    help="no benchmark: print per-dispatch counter means from a rocprofv3 --pmc CSV output "
                         "(file or directory) for the kernels matching --kernel")
    ap.add_argument("--kernel", default=".", metavar="REGEX", help="with --pmc-summary: kernel-name filter")
    a = ap.parse_args(argv)

    if a.pmc_summary:
        return pmc_summary(a.pmc_summary, a.kernel)
    if a.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (got --gpus %d)" % a.gpus)
        return 2

    import numpy as np
    import torch

    import workloads as W
    from quantized_kv_cache_encode_amd import build as kbuild

    if kbuild.is_stale():
        eprint("libkvq.so missing or stale: building")
        kbuild.build()
    import quantized_kv_cache_encode_amd.kvq as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.suite:
        run_suite(K, torch, only=a.only)
        if a.calibrate_copy:
            copy_calibration(torch)
        return 0
    if a.variant == "encode":
        return run_encode(K, torch, a)
    if a.variant == "stream":
        return run_stream(K, torch, a)
    dev = torch.device("cuda:0")
    shape = W.LONGCTX
    B, Hq, Hkv, d, T, b = shape.B, shape.Hq, shape.Hkv, shape.d, shape.T, shape.b

    eprint("generating %s: B=%d Hq=%d Hkv=%d d=%d b=%d T=%d" % (shape.name, B, Hq, Hkv, d, b, T))
    signs = W.signs(shape)
    q_np = W.queries(shape)
    keys = torch.from_numpy(W.keys(shape)).to(dev)
    v0 = torch.from_numpy(W.values(shape)).to(dev)
    newk = torch.from_numpy(W.new_keys(shape)).to(dev)
    q = torch.from_numpy(q_np).to(dev)
    pot = a.variant == "pot"
    cb = K.kvq_build_codebook_pot(d, b, 1) if pot else K.kvq_build_codebook(d, b)
    bpk = cb.bytes_per_key
    if pot:
        signs = None  # no sign pattern: the codec has no rotation

    # prefill: encode the whole cache once (setup), then make R copies at distinct addresses
    codes0 = torch.empty((B, Hkv, T, bpk), dtype=torch.uint8, device=dev)
    norms0 = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
    K.kvq_encode_keys(cb, signs, keys, codes0, norms0)
    del keys
    qv = a.variant == "qv"
    if qv:  # the values go through the same encode; the fp16 values are not kept
        vcodes0 = torch.empty_like(codes0)
        vnorms0 = torch.empty_like(norms0)
        K.kvq_encode_keys(cb, signs, v0, vcodes0, vnorms0)
        del v0
        caches = [(codes0, norms0, vcodes0, vnorms0)] + [
            (codes0.clone(), norms0.clone(), vcodes0.clone(), vnorms0.clone()) for _ in range(a.caches - 1)]
    else:
        caches = [(codes0, norms0, v0)] + [(codes0.clone(), norms0.clone(), v0.clone()) for _ in range(a.caches - 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
    ws_bytes = K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, a.splits)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)  # split-merge counters start at zero
    torch.cuda.synchronize()

    newk3 = newk[:, :, 0, :].contiguous()  # [B][Hkv][d]: the token appended on this step

    def step(i):
        if qv:
            c, n, vc, vn = caches[i % len(caches)]
            K.kvq_decode_attn_qv(cb, signs, q, c, n, vc, vn, out=out, workspace=ws, n_splits=a.splits)
            return
        c, n, v = caches[i % len(caches)]
        K.kvq_decode_attn_append(cb, signs, newk3, q, c, n, v, out=out, workspace=ws, n_splits=a.splits)

    # The steps are replayed from HIP graphs so that host-side launch overhead does not enter the timing.
    # Eager warm-up on a side stream first (the library's first launches, then the capture).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(a.warmup, len(caches))):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    g_steps = capture(step, a.steps)
    settle(torch, g_steps.replay, a.settle_seconds)  # caches, and the GPU's clocks, settle before the timed replay

    # timed region: exactly `steps` steps (one graph replay) between two synchronizations
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    g_steps.replay()
    t_stop.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    ms_per_step = total_ms / a.steps

    # a step is one launch of the fused kernel, so its mean duration is the step time: the HIP events are
    # recorded on the stream the kernels run on, around the `steps` launches of the replay
    attn_avg_ms = ms_per_step

    if a.calibrate_copy:
        copy_calibration(torch)

    key_scores = B * Hq * T
    value = key_scores / (ms_per_step * 1e-3)
    # quantized values: key and value codes + norms of every cached key, and q
    alg_bytes = (B * Hkv * T * 2 * (bpk + 4) + B * Hq * d * 2) if qv else algorithmic_bytes(shape, bpk, append=True)
    achieved = alg_bytes / (attn_avg_ms * 1e-3) / 1e9
    splits_used = ws_bytes // (B * Hq * (d + 4) * 4) if ws_bytes else 1
    eprint("step %.4f ms (one fused append + decode-attention launch)  -> %.4g key-scores/s" % (ms_per_step, value))
    eprint("decode attention: %d algorithmic bytes -> %.1f GB/s = %.1f%% of %.0f GB/s" %
           (alg_bytes, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))

    cpu = None
    if not a.no_cpu_baseline:
        eprint("timing the CPU oracle on a bounded sample (~%.0f s)" % a.cpu_seconds)
        if pot:
            cpu = cpu_baseline_pot(shape, q_np, b, 1, a.cpu_seconds)
        else:
            cpu = (cpu_baseline_qv if qv else cpu_baseline)(shape, signs, q_np, a.cpu_seconds)
        eprint("cpu oracle: %.4g key-scores/s (%s)" % (cpu["value"], cpu["sample"]))

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32 fixed-point LUT sums; fp16 P x fp16 V on MFMA with fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": "longctx decode: B=8 Hq=32 Hkv=4 d=64 b=4 T=32768, fp16 q/k/v",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "b": b, "T": T, "v_dtype": "f16",
                   "step": "one kvq_decode_attn_append launch: encode B*Hkv new keys at T-1 + decode attention over T keys",
                   "caches_rotated": len(caches), "t_splits": int(splits_used)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "decode_kernel (fused append + LUT score + online softmax + AV + split merge)",
                     "avg_launch_ms": attn_avg_ms, "algorithmic_bytes": alg_bytes},
        "cpu_baseline": cpu,
    }
    if qv:
        rec["config"].update({"workload": "longctx decode, values as 4-bit codes: B=8 Hq=32 Hkv=4 d=64 b=4 T=32768",
                              "v_dtype": "codes",
                              "step": "one kvq_decode_attn_qv launch: decode attention over T keys and values "
                                      "stored as codes + norms"})
        rec["roofline"].update({"traffic": measured_traffic(TRAFFIC_FILE_QV),
                                "kernel": "qv_decode_kernel (MFMA scores from key levels + online softmax + "
                                          "rotated-domain AV from value levels + split merge + inverse transform)"})
    if pot:
        rec["config"].update({"workload": "longctx decode, keys as 4-bit power-of-two codes with the mantissa term: "
                                          "B=8 Hq=32 Hkv=4 d=64 b=4 T=32768, fp16 q/k/v",
                              "step": "one kvq_decode_attn_append launch with a power-of-two codebook: encode B*Hkv "
                                      "new keys at T-1 + decode attention over T keys"})
        rec["roofline"].update({"traffic": None,
                                "kernel": "decode_kernel<PotScorer> (fused append + shifted-query table score + "
                                          "online softmax + AV + split merge)"})
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
