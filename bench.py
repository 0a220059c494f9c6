"""Benchmark of one tensor-parallel rank's linear share on one MI355X.

Headline (the decode half of the metric): the Llama-3.1-8B-shaped feed-forward
share at TP = 1 -- gate/up column GEMV with fused SwiGLU (4096 x 28672), down
row GEMV to an fp32 partial (14336 x 4096), and the partial sum -- for the
decode batches M = 1, 8, 32 and 64. One step runs the four batches, each on
its own copy of the layer's packed weights, so every call streams its weights
from HBM (the copies total 1.4 GB, far beyond the 256 MB last-level cache).
``value`` is algorithmic bytes / time (HBM GB/s) over the timed steps.

Secondary (the prefill half): rank 0 of TP = 8 of the Llama-3.1-405B-shaped
feed-forward layer at 8192 tokens (gate/up 16384 x 13312 + SwiGLU, down
6656 x 16384 to an fp32 partial), in bf16 TFLOP/s.

Kernel durations come from HIP events recorded on the stream the kernels run
on: around every launch in an untimed breakdown pass, and inside the timed
region around one launch of the dominant kernel per step (its launches in
turn; each recorded event costs the step a few microseconds, so no more are
recorded there). The interval of an event pair with nothing between it,
measured in the same passes, is subtracted. The other workloads (the worked
TP = 2 split, the 70B feed-forward layer at TP = 8 decode, the 70B attention
projections at prefill) are timed as whole back-to-back steps between two
events. The oracle's CPU baseline is timed on this host on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "TP-shard linear: decode HBM GB/s, prefill bf16 TFLOP/s (% of roofline)"
DECODE_MS = (1, 8, 32, 64)
COPIES = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
PREFILL_COUNTERS_FILE = os.path.join(ROOT, "profiles", "prefill_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(M, H, I, t=1):
    """Algorithmic HBM bytes of one rank's feed-forward share at batch M:
    weights once, X once, H written and read once (bf16), the fp32 partial
    written once, and the partial sum reading t partials and writing Y (at
    t = 1 the sum is taken in place, Y = P_0: nothing moves)."""
    gateup = H * 2 * (I // t) * 2 + M * H * 2 + M * (I // t) * 2
    down = (I // t) * H * 2 + M * (I // t) * 2 + M * H * 4
    reduce = (t + 1) * M * H * 4 if t > 1 else 0
    return gateup, down, reduce


def ffn_flops(M, H, I, t=1):
    return 2 * M * H * 2 * (I // t) + 2 * M * (I // t) * H


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "tensor_transformer_linear_megatron_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Timer:
    """HIP events on the stream the kernels run on, recorded with a
    device-scope release so they bracket the kernels tightly (a system-scope
    release writes back and invalidates caches at every record)."""

    FLAGS = 0x40000000  # hipEventReleaseToDevice

    def __init__(self, stream_handle):
        import ctypes
        self.ct = ctypes
        self.stream = ctypes.c_void_p(stream_handle)
        # the HIP runtime torch already loaded (the library binds to the same one)
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags({self.FLAGS:#x}) failed with {rc}")
        return e

    def record(self, e):
        if self.hip.hipEventRecord(e, self.stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value


def run_decode(args):
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl

    c = wl.LLAMA8B
    H, I = c["hidden"], c["inter"]
    log(f"[bench] generating the 8B feed-forward layer (hidden {H}, intermediate {I})")
    X = wl.activations(max(DECODE_MS), H)
    Wgu = wl.gateup(H, I, c["sigma"])
    Wd = wl.down(I, H, c["sigma"])
    gu = tp.tp_shard_plan("gateup_col", H, 2 * I, 1, 0)
    dn = tp.tp_shard_plan("row", I, H, 1, 0)
    gp0 = tp.tp_shard_pack(gu, to_dev(Wgu))
    dp0 = tp.tp_shard_pack(dn, to_dev(Wd))
    copies = [(gp0, dp0)] + [(gp0.clone(), dp0.clone()) for _ in range(COPIES - 1)]
    Xd = to_dev(X)
    bufs = {M: dict(X=Xd[:M], H=torch.empty((M, I), dtype=torch.bfloat16, device="cuda"),
                    P=torch.empty((1, M, H), dtype=torch.float32, device="cuda"),
                    ws=torch.empty(max(16, tp.tp_workspace_bytes(gu, M), tp.tp_workspace_bytes(dn, M)),
                                   dtype=torch.uint8, device="cuda")) for M in DECODE_MS}
    torch.cuda.synchronize()

    # Pre-marshalled calls of the same C entry points, so the host's launch
    # cost stays below the GPU's time per call and the stream never drains.
    import ctypes
    from tensor_transformer_linear_megatron_amd import _lib
    lib = _lib.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    VP, null = ctypes.c_void_p, ctypes.c_void_p(0)
    gub, dnb = ctypes.byref(gu), ctypes.byref(dn)
    calls = []
    for s_ in range(COPIES):
        row = []
        for j, M in enumerate(DECODE_MS):
            gp, dp = copies[(s_ * len(DECODE_MS) + j) % COPIES]
            b = bufs[M]
            ws, wsb = VP(b["ws"].data_ptr()), b["ws"].numel()
            row.append((
                (gub, VP(b["X"].data_ptr()), M, H, VP(gp.data_ptr()), VP(b["H"].data_ptr()), I, ws, wsb, stream),
                (dnb, VP(b["H"].data_ptr()), M, I, VP(dp.data_ptr()), VP(b["P"].data_ptr()), H, ws, wsb, stream),
                # t = 1: the sum of the one partial, in place (Y = P_0)
                (VP(b["P"].data_ptr()), M * H, 1, M, H, H, VP(b["P"].data_ptr()), H, stream)))
        calls.append(row)

    timer = Timer(torch.cuda.current_stream().cuda_stream)
    PARTS = ("gateup", "down", "reduce")

    def step(s, marks=None):
        """One step: every decode batch's feed-forward share. ``marks`` maps
        (M, part) to an (start, end) event pair recorded around that launch."""
        for j, M in enumerate(DECODE_MS):
            launches = zip(PARTS, (lib.tp_col_linear, lib.tp_row_linear, lib.tp_reduce_partials),
                           calls[s % COPIES][j])
            for part, fn, a in launches:
                ev = marks.get((M, part)) if marks else None
                if ev:
                    timer.record(ev[0])
                st = fn(*a)
                if ev:
                    timer.record(ev[1])
                if st:
                    raise RuntimeError(f"{part} launch failed at M={M}: {st}")

    def empty_pair(marks):
        # Two events with nothing between them: what an event pair adds to an
        # interval by itself, subtracted from the kernel intervals below.
        timer.record(marks["empty"][0])
        timer.record(marks["empty"][1])

    def new_marks(keys):
        return {k: (timer.event(), timer.event()) for k in list(keys) + ["empty"]}

    log(f"[bench] warmup {args.warmup} steps")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # Breakdown pass (untimed): every launch bracketed, to report each part
    # and to pick the dominant kernel.
    nb = min(args.steps, 20)
    bmarks = [new_marks([(M, p) for M in DECODE_MS for p in PARTS]) for _ in range(nb)]
    for s in range(nb):
        empty_pair(bmarks[s])
        step(args.warmup + s, bmarks[s])
    torch.cuda.synchronize()
    ovh_b = float(np.mean([timer.ms(*m["empty"]) for m in bmarks])) * 1e3
    per = {}
    for M in DECODE_MS:
        d = np.array([[timer.ms(*m[(M, p)]) for p in PARTS] for m in bmarks]) * 1e3 - ovh_b  # us
        gbytes, dbytes, rbytes = decode_bytes(M, H, I)
        mean = d.mean(axis=0)
        per[M] = dict(M=M, gateup_us=float(mean[0]), down_us=float(mean[1]), reduce_us=float(mean[2]),
                      gateup_GBs=gbytes / mean[0] / 1e3, down_GBs=dbytes / mean[1] / 1e3,
                      ffn_GBs=(gbytes + dbytes + rbytes) / mean.sum() / 1e3,
                      bytes=gbytes + dbytes + rbytes)
    step_bytes = sum(p["bytes"] for p in per.values())

    # The dominant kernel: the kernel symbol with the largest share of the
    # step. Batches of up to 16 tokens share one decode kernel instantiation.
    def symbol(M, part):
        if M <= 16:
            return "gemv_stream<1," + ("2,..,SwiGLU>" if part == "gateup" else "1,..,fp32>")
        return f"gemv_shared<{(M + 15) // 16},.." + (",SwiGLU>" if part == "gateup" else ",fp32>")
    groups = {}
    for M in DECODE_MS:
        gb, db, _ = decode_bytes(M, H, I)
        for part, nbytes in (("gateup", gb), ("down", db)):
            g = groups.setdefault(symbol(M, part), dict(bytes=0, us=0.0, launches=[]))
            g["bytes"] += nbytes
            g["us"] += per[M][part + "_us"]
            g["launches"].append((M, part))
    dom_name, dom = max(groups.items(), key=lambda kv: kv[1]["us"])

    # Timed region: each step brackets one launch of the dominant kernel
    # (its launches in turn) with an event pair, and every eighth step adds an
    # empty pair; every event recorded costs the step a few microseconds.
    nl = len(dom["launches"])
    tmarks = []
    for s in range(args.steps):
        m = {dom["launches"][s % nl]: (timer.event(), timer.event())}
        if s % 8 == 0:
            m["empty"] = (timer.event(), timer.event())
        tmarks.append(m)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if "empty" in tmarks[s]:
            empty_pair(tmarks[s])
        step(args.warmup + nb + s, tmarks[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = step_bytes * args.steps / wall / 1e9

    ovh = float(np.mean([timer.ms(*m["empty"]) for m in tmarks if "empty" in m])) * 1e3
    raw = float(np.mean([timer.ms(*v) for m in tmarks for k, v in m.items() if k != "empty"])) * 1e3
    avg_us = raw - ovh
    bpl = dom["bytes"] / nl
    roof = dict(bound="hbm", kernel=f"{dom_name} (decode batches M={[M for M, _ in dom['launches']]})",
                achieved=round(bpl / avg_us / 1e3, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(bpl / avg_us / 1e3 / HBM_PEAK_GBS, 4), traffic=None,
                bytes_per_launch=int(bpl), avg_launch_us=round(avg_us, 2),
                event_interval_us=round(raw, 2), empty_event_pair_us=round(ovh, 2),
                launches_per_step=nl)
    roof["traffic"] = load_traffic(dom_name, source_hash("gemv.hip"))

    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(X, Wgu, Wd, H, I)
    return dict(value=value, wall=wall, per=per, roofline=roof, cpu=cpu, H=H, I=I)


def load_traffic(key, src_hash):
    """Measured HBM bytes per launch from the committed rocprofv3 counter
    summary, or None if it is missing or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("kernels", {}).get(key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


def load_prefill_counters(workload):
    """Per-kernel MFMA utilisation, sustained clock and TFLOP/s of a prefill
    workload from the committed rocprofv3 counter summary (MfmaUtil =
    SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' active cycles), or None if it is
    missing or the GEMM source changed since the counters were taken."""
    try:
        with open(PREFILL_COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash", {}).get("gemm.hip") != source_hash("gemm.hip"):
        return None
    return t.get("workloads", {}).get(workload)


def host_cpu():
    """The host's CPU model, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(X, Wgu, Wd, H, I):
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    log(f"[bench] cpu baseline: the oracle on this host ({threads} threads)")
    sample_ms = (1, 8)
    t0 = time.perf_counter()
    reps = 0
    while True:
        for M in sample_ms:
            oracle.ffn_unsharded(X[:M], Wgu, Wd)
        reps += 1
        if time.perf_counter() - t0 > 12.0:
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes = sum(sum(decode_bytes(M, H, I)) for M in sample_ms)
    return dict(value=round(nbytes / dt / 1e9, 3), unit="GB/s", cores=threads, kind="oracle",
                sample=f"the full 8B feed-forward share (t = 1) at M = 1 and M = 8, fp64 oracle, "
                       f"{reps} repetition(s), {dt:.2f} s each; bytes counted as for the GPU",
                cpu_model=host_cpu(), nproc=os.cpu_count())


def cpu_baseline_prefill(Wgu_r, Wd_r, Hd, w, M):
    """The oracle on the same rank share (gate/up + SwiGLU, then down) for the
    first rows of the same X, in blocks of 16 rows until about 8 s have
    passed; rows are independent, so the rate carries over to all M rows."""
    import oracle
    from seeded_inputs import workloads as wl
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    log(f"[bench] cpu baseline (prefill): the oracle on this host ({threads} threads)")
    p_gu = oracle.plan("gateup_col", Hd, 2 * w, 1, 0)  # the rank's own [Wg_r | Wu_r]
    p_d = oracle.plan("row", w, Hd, 1, 0)
    rows, t0 = 0, time.perf_counter()
    while rows < M:
        Xb = wl.activations(M, Hd, rows=range(rows, rows + 16))
        oracle.row_linear(oracle.gateup_swiglu(Xb, Wgu_r, p_gu), Wd_r, p_d)
        rows += 16
        if time.perf_counter() - t0 > 8.0:
            break
    dt = time.perf_counter() - t0
    flops = rows * (2 * Hd * 2 * w + 2 * w * Hd)
    return dict(value=round(flops / dt / 1e12, 5), unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"rows 0..{rows - 1} of the 8192-token 405B rank-0 feed-forward share, fp64 oracle, "
                       f"{dt:.1f} s", cpu_model=host_cpu(), nproc=os.cpu_count())


def run_prefill(args):
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl

    c = wl.LLAMA405B
    Hd, I, t, M, r = c["hidden"], c["inter"], 8, 8192, 0
    w = I // t
    log(f"[bench] prefill: 405B feed-forward rank 0 of {t}, {M} tokens")
    cols = range(r * w, (r + 1) * w)
    X = to_dev(wl.activations(M, Hd))
    Wgu_r = wl.gateup(Hd, I, c["sigma"], cols=cols)
    Wd_r = wl.down(I, Hd, c["sigma"], rows=cols)
    gu = tp.tp_shard_plan("gateup_col", Hd, 2 * I, t, r)
    dn = tp.tp_shard_plan("row", I, Hd, t, r)
    full = torch.empty((Hd, 2 * I), dtype=torch.bfloat16, device="cuda")
    full[:, cols.start:cols.stop].copy_(to_dev(Wgu_r[:, :w]))
    full[:, I + cols.start:I + cols.stop].copy_(to_dev(Wgu_r[:, w:]))
    gp = tp.tp_shard_pack(gu, full)
    del full
    fulld = torch.empty((I, Hd), dtype=torch.bfloat16, device="cuda")
    fulld[cols.start:cols.stop].copy_(to_dev(Wd_r))
    dp = tp.tp_shard_pack(dn, fulld)
    del fulld
    Hb = torch.empty((M, w), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((M, Hd), dtype=torch.float32, device="cuda")
    for _ in range(2):
        tp.tp_col_linear(gu, X, gp, Y=Hb)
        tp.tp_row_linear(dn, Hb, dp, P=P)
    steps = max(10, args.steps // 4)
    timer = Timer(torch.cuda.current_stream().cuda_stream)
    ev = [[timer.event() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        timer.record(e[0])
        tp.tp_col_linear(gu, X, gp, Y=Hb)
        timer.record(e[1])
        tp.tp_row_linear(dn, Hb, dp, P=P)
        timer.record(e[2])
    torch.cuda.synchronize()
    # median per op over the steps (ms-scale launches: the events' own cost is negligible)
    d = np.median(np.array([[timer.ms(e[0], e[1]), timer.ms(e[1], e[2])] for e in ev]), axis=0)  # ms
    fg = 2 * M * Hd * 2 * w
    fd = 2 * M * w * Hd
    tf = (fg + fd) / d.sum() / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(Wgu_r, Wd_r, Hd, w, M)
    return dict(workload="llama3.1-405b FFN, TP=8 rank 0, prefill 8192 tokens", unit="TFLOP/s",
                value=round(tf, 1), frac=round(tf / MFMA_BF16_PEAK_TFS, 4), peak=MFMA_BF16_PEAK_TFS,
                gateup_ms=round(float(d[0]), 3), gateup_TFs=round(fg / d[0] / 1e9, 1),
                down_ms=round(float(d[1]), 3), down_TFs=round(fd / d[1] / 1e9, 1), steps=steps,
                statistic="median", mfma_counters=load_prefill_counters("405b_ffn_prefill"), cpu_baseline=cpu)


COPY_BYTES = 1 << 30


def calibrate_copy():
    """Three device-to-device copies of 1 GiB: a kernel whose HBM traffic is
    known exactly (1 GiB read, 1 GiB written per launch), run under the same
    counters as the decode kernels to scale their byte counts."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def time_steps(timer, step, n, warm=3):
    """Mean µs per step over n back-to-back steps between two events (the
    events' own cost is spread over the n steps)."""
    import torch
    for i in range(warm):
        step(i)
    e0, e1 = timer.event(), timer.event()
    torch.cuda.synchronize()
    timer.record(e0)
    for i in range(n):
        step(warm + i)
    timer.record(e1)
    torch.cuda.synchronize()
    return timer.ms(e0, e1) * 1e3 / n


def _abi():
    """The C library (already loaded by the binding) and pointer helpers, for
    pre-marshalled calls whose host cost stays below the GPU time per call."""
    import ctypes
    import torch
    from tensor_transformer_linear_megatron_amd import _lib
    lib = _lib.load()
    VP = ctypes.c_void_p
    stream = VP(torch.cuda.current_stream().cuda_stream)
    return lib, VP, ctypes.byref, stream


def _run(calls):
    for fn, a in calls:
        st = fn(*a)
        if st:
            raise RuntimeError(f"{fn.__name__} failed: {st}")


def config_worked_tp2(timer):
    """The pages' worked TP = 2 split at 8 tokens: both ranks' column and row
    shards in turn and the sum of their partials."""
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl
    lib, VP, ref, stream = _abi()
    X, W, W2 = wl.worked_tp2()
    M, H, t = X.shape[0], X.shape[1], 2
    Xd, Wd, W2d = to_dev(X), to_dev(W), to_dev(W2)
    cols = [tp.tp_shard_plan("col", H, H, t, r) for r in range(t)]
    rows = [tp.tp_shard_plan("row", H, H, t, r) for r in range(t)]
    copies = 16  # 16 x 64 MiB = 1 GiB of packed shards, far past the 256 MB last-level cache
    packs = [[(tp.tp_shard_pack(cols[r], Wd), tp.tp_shard_pack(rows[r], W2d)) for r in range(t)]
             for _ in range(copies)]
    Y = [torch.empty((M, H // t), dtype=torch.bfloat16, device="cuda") for _ in range(t)]
    P = torch.empty((t, M, H), dtype=torch.float32, device="cuda")
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    wsn = max(16, max(tp.tp_workspace_bytes(d, M) for d in cols + rows))
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda")
    steps = []
    for c in range(copies):
        calls = []
        for r in range(t):
            cp, rp = packs[c][r]
            calls.append((lib.tp_col_linear, (ref(cols[r]), VP(Xd.data_ptr()), M, H, VP(cp.data_ptr()),
                                              VP(Y[r].data_ptr()), H // t, VP(ws.data_ptr()), wsn, stream)))
            calls.append((lib.tp_row_linear, (ref(rows[r]), VP(Y[r].data_ptr()), M, H // t, VP(rp.data_ptr()),
                                              VP(P[r].data_ptr()), H, VP(ws.data_ptr()), wsn, stream)))
        calls.append((lib.tp_reduce_partials, (VP(P.data_ptr()), M * H, t, M, H, H, VP(out.data_ptr()), H, stream)))
        steps.append(calls)
    us = time_steps(timer, lambda i: _run(steps[i % copies]), 40)
    w = H * (H // t) * 2
    nbytes = t * (w + M * H * 2 + M * (H // t) * 2) + t * (w + M * (H // t) * 2 + M * H * 4) + (t + 1) * M * H * 4
    gbs = nbytes / us / 1e3
    return dict(config="worked TP=2 split: X [8 x 4096], W and W2 4096 x 4096, both ranks + sum",
                unit="GB/s", value=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4), peak=HBM_PEAK_GBS,
                us_per_step=round(us, 2), bytes_per_step=nbytes)


def decode_bytes_fp8(M, H, I, t=1):
    """Bytes one rank's feed-forward share moves with 8-bit weights: one code
    byte per weight and a 4-byte scale per output column, activations as in
    decode_bytes."""
    w = I // t
    gateup = H * 2 * w + 2 * w * 4 + M * H * 2 + M * w * 2
    down = w * H + H * 4 + M * w * 2 + M * H * 4
    return gateup, down


def config_70b_ffn_decode(timer):
    """Llama-3.1-70B feed-forward layer at TP = 8 decode: all 8 rank shares in
    turn (each gate/up + SwiGLU + down) and the sum of the 8 partials, with
    bf16 weights and with the same weights in 8-bit (OCP FP8 E4M3, one
    power-of-two scale per column; the pages' decode example is this model in
    8-bit)."""
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl
    lib, VP, ref, stream = _abi()
    c = wl.LLAMA70B
    H, I, t = c["hidden"], c["inter"], 8
    w = I // t
    log(f"[bench] 70B feed-forward at TP=8: generating [Wg | Wu] {H} x {2 * I} and Wd {I} x {H}")
    plans = {}
    for fmt in ("bf16", "fp8_e4m3"):
        plans[fmt] = ([tp.tp_shard_set_wformat(tp.tp_shard_plan("gateup_col", H, 2 * I, t, r), fmt) for r in range(t)],
                      [tp.tp_shard_set_wformat(tp.tp_shard_plan("row", I, H, t, r), fmt) for r in range(t)])
    packs = {}
    Wg = to_dev(wl.gateup(H, I, c["sigma"]))
    for fmt, (gu, _) in plans.items():
        packs[fmt] = [[tp.tp_shard_pack(d, Wg) for d in gu]]
    del Wg
    Wdn = to_dev(wl.down(I, H, c["sigma"]))
    for fmt, (_, dn) in plans.items():
        packs[fmt].append([tp.tp_shard_pack(d, Wdn) for d in dn])
    del Wdn
    X = to_dev(wl.activations(32, H))
    out_all = {}
    for fmt in ("bf16", "fp8_e4m3"):
        gu, dn = plans[fmt]
        gp, dp = packs[fmt]
        res = []
        for M in (1, 8, 32):
            Hs = torch.empty((M, w), dtype=torch.bfloat16, device="cuda")
            P = torch.empty((t, M, H), dtype=torch.float32, device="cuda")
            out = torch.empty((M, H), dtype=torch.float32, device="cuda")
            wsn = max(16, max(tp.tp_workspace_bytes(d, M) for d in gu + dn))
            ws = torch.empty(wsn, dtype=torch.uint8, device="cuda")
            calls = [(lib.tp_ffn_shard, (ref(gu[r]), ref(dn[r]), VP(X.data_ptr()), M, H, VP(gp[r].data_ptr()),
                                         VP(dp[r].data_ptr()), VP(Hs.data_ptr()), VP(P[r].data_ptr()), H,
                                         VP(ws.data_ptr()), wsn, stream)) for r in range(t)]
            calls.append((lib.tp_reduce_partials, (VP(P.data_ptr()), M * H, t, M, H, H, VP(out.data_ptr()), H,
                                                   stream)))
            us = time_steps(timer, lambda i: _run(calls), 20)
            g, d_ = decode_bytes(M, H, I, t)[:2] if fmt == "bf16" else decode_bytes_fp8(M, H, I, t)
            nbytes = t * (g + d_) + (t + 1) * M * H * 4
            gbs = nbytes / us / 1e3
            res.append(dict(M=M, us_per_step=round(us, 2), rank_share_us=round(us / t, 2), value=round(gbs, 1),
                            frac=round(gbs / HBM_PEAK_GBS, 4)))
        out_all[fmt] = res
    for a, b in zip(out_all["bf16"], out_all["fp8_e4m3"]):
        b["speedup_vs_bf16"] = round(a["us_per_step"] / b["us_per_step"], 3)
    return dict(config="llama3.1-70b FFN, TP=8 decode: 8 rank shares in turn + sum of 8 partials",
                unit="GB/s", peak=HBM_PEAK_GBS, batches=out_all["bf16"], batches_fp8_e4m3=out_all["fp8_e4m3"])


def config_70b_attention_prefill(timer):
    """Llama-3.1-70B attention projections, rank 0 of TP = 8 at 4096 tokens:
    the QKV column slice (8 Q + 1 K + 1 V head) and the O row slice."""
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl
    c = wl.LLAMA70B
    H, t, M = c["hidden"], 8, 4096
    heads = (c["n_q"], c["n_kv"], c["head_dim"])
    dq = tp.tp_shard_plan("qkv_col", H, (c["n_q"] + 2 * c["n_kv"]) * c["head_dim"], t, 0, heads=heads)
    do = tp.tp_shard_plan("o_row", c["n_q"] * c["head_dim"], H, t, 0, heads=heads)
    qp = tp.tp_shard_pack(dq, to_dev(wl.qkv_weight(H, *heads, c["sigma"])))
    op = tp.tp_shard_pack(do, to_dev(wl.o_weight(c["n_q"], c["head_dim"], H, c["sigma"])))
    X = to_dev(wl.activations(M, H))
    A = to_dev(wl.attention_output(M, c["n_q"] * c["head_dim"], cols=range(do.row_begin, do.row_end)))
    QKV = torch.empty((M, dq.out_n), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((M, H), dtype=torch.float32, device="cuda")
    tq = time_steps(timer, lambda i: tp.tp_col_linear(dq, X, qp, Y=QKV), 10)
    to_ = time_steps(timer, lambda i: tp.tp_row_linear(do, A, op, P=P), 10)
    fq, fo = 2 * M * H * dq.shard_n, 2 * M * do.shard_k * H
    tf = (fq + fo) / (tq + to_) / 1e6
    return dict(config="llama3.1-70b attention, TP=8 rank 0, prefill 4096 tokens: QKV 8192 x 1280 + O 1024 x 8192",
                unit="TFLOP/s", value=round(tf, 1), frac=round(tf / MFMA_BF16_PEAK_TFS, 4),
                peak=MFMA_BF16_PEAK_TFS, qkv_us=round(tq, 1), qkv_TFs=round(fq / tq / 1e6, 1),
                o_us=round(to_, 1), o_TFs=round(fo / to_ / 1e6, 1))


def config_sequence_parallel(timer):
    """Sequence-parallel partial sum on the 70B attention O partials of TP = 8
    at 4096 tokens ([8 x 4096 x 8192] fp32): the full rank-order sum (the
    all-reduce's arithmetic), each rank's reduce-scatter in turn, and the row
    gather of the ranks' bf16 blocks."""
    import torch
    lib, VP, ref, stream = _abi()
    t, M, N = 8, 4096, 8192
    Mt = M // t
    g = torch.Generator(device="cuda").manual_seed(0)
    P = torch.randn((t, M, N), generator=g, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Yr = torch.empty((t, Mt, N), dtype=torch.float32, device="cuda")
    Xs = torch.randn((t, Mt, N), generator=g, dtype=torch.float32, device="cuda").to(torch.bfloat16)
    X = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    full = [(lib.tp_reduce_partials, (VP(P.data_ptr()), M * N, t, M, N, N, VP(Y.data_ptr()), N, stream))]
    scatter = [(lib.tp_reduce_scatter_partials, (VP(P.data_ptr()), M * N, t, M, N, N, r,
                                                 VP(Yr[r].data_ptr()), N, stream)) for r in range(t)]
    gather = [(lib.tp_gather_rows, (VP(Xs.data_ptr()), Mt * N, t, Mt, N, N, VP(X.data_ptr()), N, stream))]
    us_full = time_steps(timer, lambda i: _run(full), 20)
    us_rs = time_steps(timer, lambda i: _run(scatter), 20)
    us_g = time_steps(timer, lambda i: _run(gather), 20)
    b_red = (t + 1) * M * N * 4  # the full sum; the t reduce-scatters move the same bytes in total
    b_g = 2 * M * N * 2
    return dict(config="sequence-parallel partial sum, 70B attention O partials at TP=8, 4096 tokens",
                unit="GB/s", peak=HBM_PEAK_GBS,
                full_sum=dict(us=round(us_full, 1), value=round(b_red / us_full / 1e3, 1),
                              frac=round(b_red / us_full / 1e3 / HBM_PEAK_GBS, 4)),
                reduce_scatter_all_ranks=dict(us=round(us_rs, 1), rank_us=round(us_rs / t, 2),
                                              value=round(b_red / us_rs / 1e3, 1),
                                              frac=round(b_red / us_rs / 1e3 / HBM_PEAK_GBS, 4)),
                gather=dict(us=round(us_g, 1), value=round(b_g / us_g / 1e3, 1),
                            frac=round(b_g / us_g / 1e3 / HBM_PEAK_GBS, 4)))


def config_70b_attention_block(timer):
    """Llama-3.1-70B attention block at TP = 8 (8 query heads and 1 key-value
    head per rank, d = 128). Decode: 32 sequences with 4096 cached positions
    each, one new token; the core alone on rank 0 (HBM GB/s of the KV cache it
    reads), and the whole block for all 8 ranks in turn (QKV slice, KV append,
    attention, O slice) plus the sum of the 8 partials; also the core at 256
    sequences. Prefill: rank 0's attention core on one 4096-token and one
    16384-token sequence (causal FLOPs)."""
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl
    lib, VP, ref, stream = _abi()
    c = wl.LLAMA70B
    H, t = c["hidden"], 8
    heads = (c["n_q"], c["n_kv"], c["head_dim"])
    d = heads[2]
    S, L = 32, 4096
    dq = [tp.tp_shard_plan("qkv_col", H, (heads[0] + 2 * heads[1]) * d, t, r, heads=heads) for r in range(t)]
    do = [tp.tp_shard_plan("o_row", heads[0] * d, H, t, r, heads=heads) for r in range(t)]
    Wq = to_dev(wl.qkv_weight(H, *heads, c["sigma"]))
    qp = [tp.tp_shard_pack(x, Wq) for x in dq]
    del Wq
    Wo = to_dev(wl.o_weight(heads[0], d, H, c["sigma"]))
    op = [tp.tp_shard_pack(x, Wo) for x in do]
    del Wo
    g = torch.Generator(device="cuda").manual_seed(70)
    caches = []
    for r in range(t):
        Kc, Vc = tp.tp_kv_cache_new(dq[r], S, L)
        Kc.copy_(torch.randn(Kc.shape, generator=g, device="cuda"))
        Vc.copy_(torch.randn(Vc.shape, generator=g, device="cuda"))
        caches.append((Kc, Vc))
    X = (torch.randn((S, H), generator=g, device="cuda")).to(torch.bfloat16)
    kv_len = torch.full((S,), L, dtype=torch.int32, device="cuda")
    slot = torch.arange(S, dtype=torch.int32, device="cuda")
    nq, w = dq[0].q_head_end - dq[0].q_head_begin, dq[0].shard_n
    QKV = torch.empty((S, w), dtype=torch.bfloat16, device="cuda")
    A = torch.empty((S, nq * d), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((t, S, H), dtype=torch.float32, device="cuda")
    out = torch.empty((S, H), dtype=torch.float32, device="cuda")
    wsn = max([tp.tp_attention_workspace_bytes(dq[0], S, 1, L)] + [tp.tp_workspace_bytes(x, S) for x in dq + do] + [16])
    ws = torch.empty(wsn, dtype=torch.uint8, device="cuda")
    KL, SLP = VP(kv_len.data_ptr()), VP(slot.data_ptr())

    def attn_call(r):
        Kc, Vc = caches[r]
        return (lib.tp_attention, (ref(dq[r]), VP(QKV.data_ptr()), w, S, 1, KL, SLP, L, VP(Kc.data_ptr()),
                                   VP(Vc.data_ptr()), S, L, VP(A.data_ptr()), nq * d, VP(ws.data_ptr()), wsn, stream))

    block = []
    for r in range(t):
        Kc, Vc = caches[r]
        block += [(lib.tp_col_linear, (ref(dq[r]), VP(X.data_ptr()), S, H, VP(qp[r].data_ptr()), VP(QKV.data_ptr()), w,
                                       VP(ws.data_ptr()), wsn, stream)),
                  (lib.tp_kv_append, (ref(dq[r]), VP(QKV.data_ptr()), w, S, 1, KL, SLP, VP(Kc.data_ptr()),
                                      VP(Vc.data_ptr()), S, L, stream)),
                  attn_call(r),
                  (lib.tp_row_linear, (ref(do[r]), VP(A.data_ptr()), S, nq * d, VP(op[r].data_ptr()),
                                       VP(P[r].data_ptr()), H, VP(ws.data_ptr()), wsn, stream))]
    block.append((lib.tp_reduce_partials, (VP(P.data_ptr()), S * H, t, S, H, H, VP(out.data_ptr()), H, stream)))
    _run(block)
    core = [attn_call(0)]
    us_core = time_steps(timer, lambda i: _run(core), 20)
    us_block = time_steps(timer, lambda i: _run(block), 10)
    kv_bytes = S * L * 1 * d * 2 * 2  # one key-value head per rank
    core_bytes = kv_bytes + S * w * 2 + S * nq * d * 2
    wq, wo = H * w * 2, nq * d * H * 2
    block_bytes = t * (wq + wo + kv_bytes + S * H * 2 + S * w * 2 * 2 + S * nq * d * 2 * 2) + (t + 1) * S * H * 4
    # prefill core, rank 0, one 4096-token sequence
    T = 4096
    Kp, Vp = tp.tp_kv_cache_new(dq[0], 1, T)
    QKVp = (torch.randn((T, w), generator=g, device="cuda")).to(torch.bfloat16)
    Ap = torch.empty((T, nq * d), dtype=torch.bfloat16, device="cuda")
    klp = torch.full((1,), T, dtype=torch.int32, device="cuda")
    slp = torch.zeros((1,), dtype=torch.int32, device="cuda")
    tp.tp_kv_append(dq[0], QKVp, T, klp, slp, Kp, Vp)
    pre = [(lib.tp_attention, (ref(dq[0]), VP(QKVp.data_ptr()), w, 1, T, VP(klp.data_ptr()), VP(slp.data_ptr()), T,
                               VP(Kp.data_ptr()), VP(Vp.data_ptr()), 1, T, VP(Ap.data_ptr()), nq * d, VP(0), 0,
                               stream))]
    us_pre = time_steps(timer, lambda i: _run(pre), 10)
    flops = 4 * nq * d * T * (T + 1) // 2
    del Kp, Vp, QKVp, Ap, caches
    # decode core at a serving batch (256 sequences x 4096 positions: one
    # 4096-position chunk per workgroup, no merge) and the prefill core on one
    # 16384-token sequence (the two-group form)
    S2 = 256
    K2, V2 = tp.tp_kv_cache_new(dq[0], S2, L)
    K2.copy_(torch.randn(K2.shape, generator=g, device="cuda"))
    V2.copy_(torch.randn(V2.shape, generator=g, device="cuda"))
    Q2 = (torch.randn((S2, w), generator=g, device="cuda")).to(torch.bfloat16)
    A2 = torch.empty((S2, nq * d), dtype=torch.bfloat16, device="cuda")
    kl2 = torch.full((S2,), L, dtype=torch.int32, device="cuda")
    sl2 = torch.arange(S2, dtype=torch.int32, device="cuda")
    ws2n = max(16, tp.tp_attention_workspace_bytes(dq[0], S2, 1, L))
    ws2 = torch.empty(ws2n, dtype=torch.uint8, device="cuda")
    big = [(lib.tp_attention, (ref(dq[0]), VP(Q2.data_ptr()), w, S2, 1, VP(kl2.data_ptr()), VP(sl2.data_ptr()), L,
                               VP(K2.data_ptr()), VP(V2.data_ptr()), S2, L, VP(A2.data_ptr()), nq * d,
                               VP(ws2.data_ptr()), ws2n, stream))]
    us_big = time_steps(timer, lambda i: _run(big), 20)
    big_bytes = S2 * L * d * 2 * 2 + S2 * w * 2 + S2 * nq * d * 2
    del K2, V2
    T2 = 16384
    Kq, Vq = tp.tp_kv_cache_new(dq[0], 1, T2)
    Qq = (torch.randn((T2, w), generator=g, device="cuda")).to(torch.bfloat16)
    Aq = torch.empty((T2, nq * d), dtype=torch.bfloat16, device="cuda")
    klq = torch.full((1,), T2, dtype=torch.int32, device="cuda")
    tp.tp_kv_append(dq[0], Qq, T2, klq, slp, Kq, Vq)
    long_pre = [(lib.tp_attention, (ref(dq[0]), VP(Qq.data_ptr()), w, 1, T2, VP(klq.data_ptr()), VP(slp.data_ptr()),
                                    T2, VP(Kq.data_ptr()), VP(Vq.data_ptr()), 1, T2, VP(Aq.data_ptr()), nq * d,
                                    VP(0), 0, stream))]
    us_long = time_steps(timer, lambda i: _run(long_pre), 5)
    flops_long = 4 * nq * d * T2 * (T2 + 1) // 2
    return dict(config="llama3.1-70b attention, TP=8 (8 query heads + 1 KV head per rank, d=128)",
                decode=dict(batch=S, context=L,
                            core_rank0=dict(us=round(us_core, 2), kv_bytes=kv_bytes,
                                            value=round(core_bytes / us_core / 1e3, 1), unit="GB/s",
                                            frac=round(core_bytes / us_core / 1e3 / HBM_PEAK_GBS, 4)),
                            block_8_ranks=dict(us=round(us_block, 1), bytes=block_bytes,
                                               value=round(block_bytes / us_block / 1e3, 1), unit="GB/s",
                                               frac=round(block_bytes / us_block / 1e3 / HBM_PEAK_GBS, 4))),
                decode_core_rank0_batch256=dict(batch=S2, context=L, us=round(us_big, 2),
                                                value=round(big_bytes / us_big / 1e3, 1), unit="GB/s",
                                                frac=round(big_bytes / us_big / 1e3 / HBM_PEAK_GBS, 4)),
                prefill_core_rank0=dict(tokens=T, us=round(us_pre, 1), flops=flops,
                                        value=round(flops / us_pre / 1e6, 1), unit="TFLOP/s",
                                        frac=round(flops / us_pre / 1e6 / MFMA_BF16_PEAK_TFS, 4)),
                prefill_core_rank0_16384=dict(tokens=T2, us=round(us_long, 1), flops=flops_long,
                                              value=round(flops_long / us_long / 1e6, 1), unit="TFLOP/s",
                                              frac=round(flops_long / us_long / 1e6 / MFMA_BF16_PEAK_TFS, 4)))


def config_405b_ffn_backward(timer):
    """Backward of rank 0's Llama-3.1-405B feed-forward share at TP = 8 and
    8192 tokens (the prefill workload above): dH through the down projection's
    transposed shard, the SwiGLU gradient, dX_0 through the gate/up transposed
    shard, and the two weight gradients; saved activations X, [G | U], H and
    the output gradient dY are resident."""
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl
    c = wl.LLAMA405B
    Hd, I, t, M, r = c["hidden"], c["inter"], 8, 8192, 0
    w = I // t
    gu = tp.tp_shard_plan("gateup_col", Hd, 2 * I, t, r)
    dn = tp.tp_shard_plan("row", I, Hd, t, r)
    dgu, ddn = tp.tp_shard_plan_dgrad(gu), tp.tp_shard_plan_dgrad(dn)
    g = torch.Generator(device="cuda").manual_seed(405)

    def randn(shape, sigma, dtype=torch.bfloat16):
        return (torch.randn(shape, generator=g, dtype=torch.float32, device="cuda") * sigma).to(dtype)

    full = torch.empty((Hd, 2 * I), dtype=torch.bfloat16, device="cuda")
    full[:, r * w:(r + 1) * w] = randn((Hd, w), c["sigma"])
    full[:, I + r * w:I + (r + 1) * w] = randn((Hd, w), c["sigma"])
    gp = tp.tp_shard_pack(dgu, full)
    del full
    fulld = torch.empty((I, Hd), dtype=torch.bfloat16, device="cuda")
    fulld[r * w:(r + 1) * w] = randn((w, Hd), c["sigma"])
    dp = tp.tp_shard_pack(ddn, fulld)
    del fulld
    X, dY = randn((M, Hd), 1.0), randn((M, Hd), 1.0)
    GU, H = randn((M, 2 * w), 1.0), randn((M, w), 0.5)
    dH = torch.empty((M, w), dtype=torch.float32, device="cuda")
    dGU = torch.empty((M, 2 * w), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, Hd), dtype=torch.float32, device="cuda")
    dWgu = torch.empty((Hd, 2 * w), dtype=torch.float32, device="cuda")
    dWd = torch.empty((w, Hd), dtype=torch.float32, device="cuda")
    us = dict(dgrad_down=time_steps(timer, lambda i: tp.tp_row_linear(ddn, dY, dp, P=dH), 5),
              swiglu_bwd=time_steps(timer, lambda i: tp.tp_swiglu_backward(GU, dH, dGU=dGU), 10),
              dgrad_gateup=time_steps(timer, lambda i: tp.tp_row_linear(dgu, dGU, gp, P=dX), 5),
              wgrad_gateup=time_steps(timer, lambda i: tp.tp_weight_grad(gu, X, dGU, dW=dWgu), 5),
              wgrad_down=time_steps(timer, lambda i: tp.tp_weight_grad(dn, H, dY, dW=dWd), 5))
    fl = dict(dgrad_down=2 * M * Hd * w, dgrad_gateup=2 * M * 2 * w * Hd, wgrad_gateup=2 * M * Hd * 2 * w,
              wgrad_down=2 * M * w * Hd)
    total = sum(fl.values()) / sum(us.values()) / 1e6
    sw_bytes = M * w * (2 * 2 + 4 + 2 * 2)
    per = {k: dict(us=round(v, 1), **({"TFLOP/s": round(fl[k] / v / 1e6, 1)} if k in fl else
                                       {"GB/s": round(sw_bytes / v / 1e3, 1)}))
           for k, v in us.items()}
    return dict(config="llama3.1-405b FFN backward, TP=8 rank 0, 8192 tokens: dgrad + wgrad of gate/up "
                       "16384 x 13312 and down 6656 x 16384, SwiGLU gradient",
                unit="TFLOP/s", value=round(total, 1), frac=round(total / MFMA_BF16_PEAK_TFS, 4),
                peak=MFMA_BF16_PEAK_TFS, per_op=per)


def config_8b_ffn_batches(timer):
    """The Llama-3.1-8B feed-forward share at TP = 1 between decode and full
    prefill: batches of 96 to 1024 tokens, gate/up + SwiGLU and down timed
    apart on 4 rotating weight copies (1.4 GB), in GB/s of the algorithmic
    bytes and TFLOP/s. Up to 512 tokens the products run the 128-token-tile
    GEMM, beyond it the 256-token one."""
    import torch
    import tensor_transformer_linear_megatron_amd as tp
    from seeded_inputs import workloads as wl
    lib, VP, ref, stream = _abi()
    c = wl.LLAMA8B
    H, I = c["hidden"], c["inter"]
    gu = tp.tp_shard_plan("gateup_col", H, 2 * I, 1, 0)
    dn = tp.tp_shard_plan("row", I, H, 1, 0)
    log("[bench] 8B feed-forward share: generating and packing 4 weight copies")
    Wg, Wd = to_dev(wl.gateup(H, I, c["sigma"])), to_dev(wl.down(I, H, c["sigma"]))
    packs = [(tp.tp_shard_pack(gu, Wg), tp.tp_shard_pack(dn, Wd)) for _ in range(4)]
    del Wg, Wd
    Ms = (96, 128, 256, 384, 512, 768, 1024)
    X = to_dev(wl.activations(max(Ms), H))
    res = []
    for M in Ms:
        Hs = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
        P = torch.empty((M, H), dtype=torch.float32, device="cuda")
        wsn = max(16, tp.tp_workspace_bytes(gu, M), tp.tp_workspace_bytes(dn, M))
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda")
        g_calls = [[(lib.tp_col_linear, (ref(gu), VP(X.data_ptr()), M, H, VP(gp.data_ptr()), VP(Hs.data_ptr()), I,
                                         VP(ws.data_ptr()), wsn, stream))] for gp, _ in packs]
        d_calls = [[(lib.tp_row_linear, (ref(dn), VP(Hs.data_ptr()), M, I, VP(dp.data_ptr()), VP(P.data_ptr()), H,
                                         VP(ws.data_ptr()), wsn, stream))] for _, dp in packs]
        ug = time_steps(timer, lambda i: _run(g_calls[i % 4]), 20)
        ud = time_steps(timer, lambda i: _run(d_calls[i % 4]), 20)
        gb, db, _ = decode_bytes(M, H, I)
        fl_g, fl_d = 2 * M * H * 2 * I, 2 * M * I * H
        res.append(dict(M=M, gateup_us=round(ug, 2), down_us=round(ud, 2), gateup_GBs=round(gb / ug / 1e3, 1),
                        down_GBs=round(db / ud / 1e3, 1), gateup_TFs=round(fl_g / ug / 1e6, 1),
                        down_TFs=round(fl_d / ud / 1e6, 1)))
    return dict(config="llama3.1-8b FFN share, TP=1, batches of 96-1024 tokens", unit="GB/s and TFLOP/s",
                batches=res)


def config_405b_ffn_prefill(timer):
    """The prefill workload alone (rank 0 of the 405B feed-forward layer at
    TP = 8, 8192 tokens), without the CPU baseline: for profiler runs."""
    return run_prefill(argparse.Namespace(steps=40, no_cpu_baseline=True))


CONFIGS = {"worked_tp2": config_worked_tp2, "70b_ffn_decode": config_70b_ffn_decode,
           "70b_attention_prefill": config_70b_attention_prefill, "sequence_parallel": config_sequence_parallel,
           "405b_ffn_backward": config_405b_ffn_backward, "70b_attention_block": config_70b_attention_block}
# run only with --config (the default line already carries the prefill workload)
PROFILE_ONLY = {"405b_ffn_prefill": config_405b_ffn_prefill, "8b_ffn_batches": config_8b_ffn_batches}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (worked TP=2 split, 70B decode and attention prefill, "
                         "sequence-parallel partial sum, 405B feed-forward backward, 70B attention block)")
    ap.add_argument("--config", choices=sorted({**CONFIGS, **PROFILE_ONLY}),
                    help="only run this one workload and print its line (for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (the yardstick for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every tensor-parallel rank runs in turn on a single MI355X "
              "and there is no multi-GPU path; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.config:
        timer = Timer(torch.cuda.current_stream().cuda_stream)
        print(json.dumps({**CONFIGS, **PROFILE_ONLY}[args.config](timer)), flush=True)
        return
    dec = run_decode(args)
    pre = None if args.no_prefill else run_prefill(args)
    others = None
    if not args.no_configs:
        timer = Timer(torch.cuda.current_stream().cuda_stream)
        others = [fn(timer) for fn in CONFIGS.values()]
    per = [dict(M=p["M"], gateup_us=round(p["gateup_us"], 2), down_us=round(p["down_us"], 2),
                reduce_us=round(p["reduce_us"], 2), gateup_GBs=round(p["gateup_GBs"], 1),
                down_GBs=round(p["down_GBs"], 1), ffn_GBs=round(p["ffn_GBs"], 1))
           for p in dec["per"].values()]
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights, random init)",
        "config": {"workload": "llama3.1-8b FFN share, TP=1, decode batches M=1,8,32,64 per step",
                   "hidden": dec["H"], "intermediate": dec["I"], "t": 1,
                   "decode_batches": list(DECODE_MS), "weight_copies": COPIES,
                   "frac_of_hbm_peak": round(dec["value"] / HBM_PEAK_GBS, 4)},
        "roofline": dec["roofline"],
        "cpu_baseline": dec["cpu"],
        "per_batch": per,
        "prefill": pre,
        "other_configs": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
