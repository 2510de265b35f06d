"""Benchmark of the slot-indexed Gated DeltaNet state path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  `value` is the decode step's algorithmic HBM traffic
per second (GB/s) on the decode workload: 256 rows x 1 token, 32 v-heads /
16 k-heads, 128x128 fp32 state per head, 8192 bf16 conv channels with 4
taps, 1024-slot pool with pages padded to 4 KiB, 90 % of the rows warm.
Alongside: varlen prefill tokens/s (8 sequences of U{512..4096} tokens, 16
heads; also 64 x 1000 tokens at 32 heads) with its flop rate against the fp32
vector peak, and the cross-layer restore GB/s (48 GDN layers of a 64-layer
stack, 64 ops, a quarter of them misses).  Inputs are synthetic and resident
in HBM before timing; timing uses HIP events on the stream the kernels run
on: `value` comes from K decode steps between one pair of events, the
per-launch percentiles and the secondary figures from one pair per call.
The CPU baseline is the oracle timed on this host on the same decode batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X published fp32 vector peak (packed FMA)
FP32_NONPACKED_PEAK_TFLOPS = 78.6  # the same without packed FMA, which this build does not emit

METRIC = "GDN decode state GB/s (% HBM peak) + prefill tokens/s, 32 heads x 128x128 fp32"


def decode_bytes(inp) -> int:
    """Algorithmic bytes of one decode step: state read for warm rows and
    written for all rows, window read (warm) and written, x, alpha, beta,
    output, conv weights (and bias), state index and flag."""
    g = inp.geom
    B = inp.num_seqs
    n_w = int(inp.has_initial_state.sum())
    tile = g.Hv * g.dk * g.dv * 4
    win = (g.W - 1) * g.C * 2
    bias = g.C * 2 if inp.conv_b is not None else 0
    return (n_w * tile + B * tile + n_w * win + B * win + B * g.C * 2 + B * g.Hv * 8
            + B * g.Hv * g.dv * 2 + g.C * g.W * 2 + bias + 5 * B)


def prefill_bytes(inp) -> int:
    """Algorithmic bytes of one varlen prefill: x, alpha, beta and output of
    every token, each sequence's state and window read (warm) and written,
    conv weights (and bias), slot index, flag and the n + 1 offsets."""
    g = inp.geom
    T = inp.total_tokens
    n = inp.num_seqs
    n_w = int(inp.has_initial_state.sum())
    tile = g.Hv * g.dk * g.dv * 4
    win = (g.W - 1) * g.C * 2
    bias = g.C * 2 if inp.conv_b is not None else 0
    return (T * g.C * 2 + T * g.Hv * 8 + T * g.Hv * g.dv * 2 + (n_w + n) * (tile + win)
            + g.C * g.W * 2 + bias + 9 * n + 4)


DECODE_SOURCES = ("hybrid_linear_attention_slot_amd/csrc/decode_kernel.hip",
                  "hybrid_linear_attention_slot_amd/csrc/device_utils.h")
DECODE_PROFILE = "profiles/decode_kernel_256rows_32heads_128x128.md"


def measured_traffic(profile: str, sources) -> "int | None":
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary of
    the kernel, or None when the kernel sources have changed since the
    counters were taken (the summary records the sources' sha256)."""
    import hashlib
    path = os.path.join(ROOT, profile)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for s in sources:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    nbytes = digest = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic_bytes_per_launch:"):
                nbytes = int(line.split(":")[1])
            elif line.startswith("source_sha256:"):
                digest = line.split(":")[1].split()[0]
    return nbytes if digest == h.hexdigest() else None


def prefill_flops(inp) -> int:
    """Algorithmic flops: per token, 6 dk dv per v-head (decay, S k, rank-1
    update, S q as multiply-adds) and 2 W per conv channel."""
    g = inp.geom
    return inp.total_tokens * (g.Hv * 6 * g.dk * g.dv + 2 * g.W * g.C)


def per_call(fn, n, stream):
    """Each of n calls bracketed by its own pair of events: p10 / p50 / p90 in ms."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.sort([a.elapsed_time(b) for a, b in ev])
    return {"p10": float(np.percentile(t, 10)), "p50": float(np.percentile(t, 50)),
            "p90": float(np.percentile(t, 90))}


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per call


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def bench_decode(steps, warmup, extra_pad=0):
    import torch
    import hybrid_linear_attention_slot_amd as gdn
    import workloads as wl

    inp, pages = wl.decode_workload(seed=0, extra_pad=extra_pad)
    g = inp.geom
    pool = torch.zeros((g.num_slots, g.page_stride), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(inp.state_indices.astype(np.int64)).cuda()
    pool[idx] = torch.from_numpy(pages).cuda()
    h = gdn.gdn_pool_create([pool], g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                            g.W, g.Hk, g.Hv, g.dk, g.dv)
    out = torch.empty((inp.num_seqs, g.Hv, g.dv), dtype=torch.int16, device="cuda")
    args = gdn.make_step_args(dev(inp.x), dev(inp.conv_w), None, dev(inp.alpha), dev(inp.beta),
                              dev(inp.state_indices), dev(inp.has_initial_state), out, 1.0, 1e-6)
    stream = torch.cuda.current_stream()
    step = lambda: gdn.gdn_decode_step(h, 0, inp.num_seqs, args, stream)  # noqa: E731
    ms = timed(step, steps, warmup, stream)
    return inp, ms, decode_bytes(inp), per_call(step, steps, stream)


def bench_prefill(steps, warmup, with_checkpoints=True):
    import torch
    import hybrid_linear_attention_slot_amd as gdn
    import workloads as wl

    inp, img = wl.prefill_workload(seed=0)
    g = inp.geom
    pool = dev(img)
    h = gdn.gdn_pool_create([pool], g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                            g.W, g.Hk, g.Hv, g.dk, g.dv)
    out = torch.empty((inp.total_tokens, g.Hv, g.dv), dtype=torch.int16, device="cuda")
    args = gdn.make_step_args(dev(inp.x), dev(inp.conv_w), None, dev(inp.alpha), dev(inp.beta),
                              dev(inp.state_indices), dev(inp.has_initial_state), out, 1.0, 1e-6)
    cu = dev(inp.cu_seqlens)
    stream = torch.cuda.current_stream()
    call = lambda: gdn.gdn_prefill_varlen(h, 0, inp.num_seqs, cu, inp.max_seqlen,  # noqa: E731
                                          inp.total_tokens, args, stream)
    timed(call, 1, max(1, warmup), stream)
    pc = per_call(call, max(2, steps), stream)
    if not with_checkpoints:
        return inp, pc, None
    # the same call emitting every sequence's state at its last 256-token block
    # boundary into a spare slot
    lens = np.diff(inp.cu_seqlens)
    used = set(inp.state_indices.tolist())
    ck_slot = dev(np.array([s for s in range(g.num_slots) if s not in used][:inp.num_seqs],
                           np.int32))
    ck_len = dev((lens // 256 * 256).astype(np.int32))
    ck = per_call(lambda: gdn.gdn_prefill_varlen_checkpoint(h, 0, inp.num_seqs, cu,
                                                            inp.max_seqlen, inp.total_tokens,
                                                            args, ck_slot, ck_len, stream),
                  max(2, steps), stream)
    return inp, pc, ck["p50"]


def bench_prefill_32heads(steps, warmup, n_seq=64, seq_len=1000):
    """Prefill at the decode geometry (32 v-heads / 16 k-heads, 8192 channels):
    64 sequences of 1000 tokens from a cold start, inputs drawn on the device."""
    import torch
    import hybrid_linear_attention_slot_amd as gdn
    import workloads as wl

    g = wl.decode_geometry(num_slots=n_seq)
    pool = torch.zeros((g.num_slots, g.page_stride), dtype=torch.uint8, device="cuda")
    h = gdn.gdn_pool_create([pool], g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C,
                            g.W, g.Hk, g.Hv, g.dk, g.dv)
    gen = wl.device_generator(32, n_seq, seq_len)
    T = n_seq * seq_len
    x = wl.device_x(gen, T, g.C)
    alpha, beta = wl.device_gates(gen, T, g.Hv)
    rng = wl.rng_for(32)
    w, _ = wl.draw_conv_params(rng, g.C, g.W, bias=False)
    out = torch.empty((T, g.Hv, g.dv), dtype=torch.int16, device="cuda")
    idx = torch.arange(n_seq, dtype=torch.int32, device="cuda")
    hs = torch.zeros(n_seq, dtype=torch.uint8, device="cuda")
    args = gdn.make_step_args(x, dev(w), None, alpha, beta, idx, hs, out, 1.0, 1e-6)
    cu = torch.arange(0, T + 1, seq_len, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: gdn.gdn_prefill_varlen(h, 0, n_seq, cu, seq_len, T, args, stream)  # noqa: E731
    timed(call, 1, max(1, warmup // 2), stream)
    pc = per_call(call, max(2, steps // 5), stream)
    del pool, x, out
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(T / (pc["p50"] * 1e-3), 1), "ms_per_call": round(pc["p50"], 4),
            "workload": f"{n_seq} seqs x {seq_len} tokens, 32 v-heads/16 k-heads, 128x128 fp32, "
                        "cold start (the continuation run's shape)"}


def bench_restore(steps, warmup):
    import torch
    import hybrid_linear_attention_slot_amd as gdn
    import workloads as wl

    g, linear, ops = wl.restore_workload(seed=0)
    bufs = [torch.empty((g.num_slots, g.page_stride), dtype=torch.uint8, device="cuda")
            if lin else None for lin in linear]
    h = gdn.gdn_pool_create(bufs, g.num_slots, g.page_stride, g.conv_off, g.ssm_off, g.C, g.W,
                            g.Hk, g.Hv, g.dk, g.dv)
    hs = torch.ones(len(ops), dtype=torch.uint8, device="cuda")
    op_list = ops.tolist()
    stream = torch.cuda.current_stream()
    call = lambda: gdn.gdn_restore_slots(h, op_list, hs, stream)  # noqa: E731
    timed(call, 1, max(1, warmup), stream)
    ms = per_call(call, max(2, steps), stream)["p50"]
    hits = int((ops[:, 1] >= 0).sum())
    payload = g.ssm_region_bytes + g.conv_region_bytes
    nbytes = 2 * hits * int(linear.sum()) * payload
    # gather / scatter of the 64 op rows' pages on every GDN layer (one launch
    # per layer, 48 launches per timed call).  Every layer has dense rows of its
    # own (6.6 GB in all): with one shared 137 MB pair the dense side of every
    # call after the first could be served from the GPU's 256 MB last-level
    # cache instead of HBM.
    idx = torch.from_numpy(np.ascontiguousarray(ops[:, 0])).cuda()
    n = idx.numel()
    layers = [l for l, lin in enumerate(linear) if lin]
    ssm = [torch.empty((n, g.ssm_region_bytes), dtype=torch.uint8, device="cuda") for _ in layers]
    conv = [torch.empty((n, g.conv_region_bytes), dtype=torch.uint8, device="cuda") for _ in layers]
    gather = lambda: [gdn.gdn_gather_states(h, l, idx, n, conv[i], ssm[i], stream)  # noqa: E731
                      for i, l in enumerate(layers)]
    scatter = lambda: [gdn.gdn_scatter_states(h, l, idx, n, conv[i], ssm[i], stream)  # noqa: E731
                       for i, l in enumerate(layers)]
    gs_bytes = 2 * n * len(layers) * payload
    gs = {}
    for name, fn in (("gather", gather), ("scatter", scatter)):
        timed(fn, 1, 1, stream)
        gms = per_call(fn, 5, stream)["p50"]
        gs[name] = {"gb_per_s": round(gs_bytes / (gms * 1e-3) / 1e9, 2), "ms_per_call": round(gms, 4),
                    "frac_of_hbm_peak": round(gs_bytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    gs["bytes"] = gs_bytes
    gs["what"] = f"{n} pages of each of the {len(layers)} GDN layers to dense rows and back " \
                 "(one launch per layer, each layer with dense rows of its own; median of 5 " \
                 "per-call events over all layers)"
    del ssm, conv
    snap = bench_snapshot(h, int(ops[0, 0]), int(ops[1, 0]), int(linear.sum()) * payload)
    del bufs
    torch.cuda.empty_cache()
    return ms, nbytes, hits, int(linear.sum()), snap, gs


def bench_snapshot(pool, slot_a, slot_b, payload, reps=3):
    """Save one slot (every GDN layer) to a snapshot file and load it into
    another slot, host time including the device copies, CRC-32C and file I/O."""
    import tempfile

    import hybrid_linear_attention_slot_amd as gdn
    d = tempfile.mkdtemp(prefix="gdn_snap_")
    path = os.path.join(d, "slot.snap")
    t_save = t_load = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        gdn.gdn_snapshot_save(pool, slot_a, 1, 0, path)
        t1 = time.perf_counter()
        gdn.gdn_snapshot_load(pool, slot_b, path, 1)
        t2 = time.perf_counter()
        t_save += t1 - t0
        t_load += t2 - t1
    os.remove(path)
    os.rmdir(d)
    return {"payload_bytes": payload, "save_ms": round(t_save / reps * 1e3, 2),
            "load_ms": round(t_load / reps * 1e3, 2),
            "save_gb_per_s": round(payload / (t_save / reps) / 1e9, 3),
            "load_gb_per_s": round(payload / (t_load / reps) / 1e9, 3),
            "where": d.rsplit("/", 1)[0]}


def bench_slot_manager(rows=256, steps=200):
    """Host cost of one scheduler step of the slot manager: resolve + commit of
    a 256-row batch in which every row asks for a restore and a save.  The
    request arrays are built beforehand; the timed loop makes only the two
    C-ABI calls per step."""
    import ctypes

    import hybrid_linear_attention_slot_amd as gdn
    L = gdn.lib()
    m = gdn.gdn_slots_create(4 * rows, 16)
    for q in range(rows):
        gdn.gdn_slots_add_sequence(m, q)
    reqs = []
    for st in range(steps):
        arr = (gdn.gdn_slot_request * rows)(
            *[gdn.gdn_slot_request(q, 16 * st, 16 * st + 16, (st << 20) + q + 1,
                                   ((st + 1) << 20) + q + 1) for q in range(rows)])
        reqs.append(arr)
    ops = (gdn.gdn_linear_state_op * rows)()
    t0 = time.perf_counter()
    for arr in reqs:
        if L.gdn_slots_resolve(m.handle, arr, rows, ops) != 0 or L.gdn_slots_commit(m.handle) != 0:
            raise RuntimeError(gdn.gdn_last_error())
    dt = time.perf_counter() - t0
    gdn.gdn_slots_destroy(m)
    return {"us_per_step": round(dt / steps * 1e6, 2), "rows": rows,
            "note": "resolve + commit (C-ABI calls only) of 256 rows that all request a "
                    "save and a restore; 1024 slots, so the first steps promote every row "
                    "and later ones match restores and skip saves for want of free slots"}


def bench_copy(reps=10):
    """Context for the HBM-bound rows: torch's device-to-device copy of 1 GiB
    (read + write bytes counted), median of per-call events."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    pc = per_call(lambda: dst.copy_(src), reps, st)
    del src, dst
    torch.cuda.empty_cache()
    return {"gb_per_s": round(2 * n / (pc["p50"] * 1e-3) / 1e9, 2), "bytes_per_call": 2 * n,
            "what": "torch copy_ of a 1 GiB device buffer (read + write), median of "
                    f"{reps} per-call events"}


def bench_ceilings(reps=10):
    """HBM ceilings on this GPU for the path's access patterns (the kernels of
    libgdn_ceilings.so: no arithmetic, only the bytes): a 2 GiB read-only
    stream, a 2 GiB write-only stream, and the decode's pattern, an in-place
    read-modify-write of the 2 MiB state region of 256 scattered pages of a
    1024-page pool with the decode's page stride.  Median of per-call events."""
    import ctypes

    import torch
    import workloads as wl

    lib = ctypes.CDLL(os.path.join(ROOT, "hybrid_linear_attention_slot_amd",
                                   "libgdn_ceilings.so"))
    p, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    lib.gdnc_read.argtypes = [p, i64, p, p]
    lib.gdnc_write.argtypes = [p, i64, u32, p]
    lib.gdnc_rmw.argtypes = [p, i64, p, i32, i64, p]
    lib.gdnc_copy.argtypes = [p, p, i64, p]
    st = torch.cuda.current_stream()
    sp = st.cuda_stream
    n = 2 << 30
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(n // (128 << 10), dtype=torch.int32, device="cuda")

    def run(fn):
        for _ in range(2):
            assert fn() == 0
        return per_call(lambda: fn(), reps, st)["p50"]

    rd = run(lambda: lib.gdnc_read(buf.data_ptr(), n, sink.data_ptr(), sp))
    wr = run(lambda: lib.gdnc_write(buf.data_ptr(), n, 7, sp))
    half = n // 2  # 1 GiB into the other 1 GiB
    cp = run(lambda: lib.gdnc_copy(buf.data_ptr(), buf.data_ptr() + half, half, sp))
    del buf, sink
    inp, _ = wl.decode_workload(seed=0)
    g = inp.geom
    assert g.ssm_off == 0 and g.ssm_region_bytes == 2 << 20
    pool = torch.ones((g.num_slots, g.page_stride), dtype=torch.uint8, device="cuda")
    pages = dev(inp.state_indices)
    nb = 2 * inp.num_seqs * g.ssm_region_bytes
    rmw = run(lambda: lib.gdnc_rmw(pool.data_ptr(), g.page_stride, pages.data_ptr(),
                                   inp.num_seqs, g.ssm_region_bytes, sp))
    del pool
    torch.cuda.empty_cache()
    return {"read_gb_per_s": round(n / (rd * 1e-3) / 1e9, 1),
            "write_gb_per_s": round(n / (wr * 1e-3) / 1e9, 1),
            "rmw_gb_per_s": round(nb / (rmw * 1e-3) / 1e9, 1),
            "copy_gb_per_s": round(2 * half / (cp * 1e-3) / 1e9, 1),
            "what": "libgdn_ceilings kernels: 2 GiB read-only and write-only streams, a copy "
                    "of 1 GiB into another (read + write bytes), and the in-place "
                    "read-modify-write of the 2 MiB state region of the decode workload's 256 "
                    "pages (read + write bytes); 1024-thread workgroups, 128 KiB each, "
                    "non-temporal (the read-modify-write's stores at device scope, SC1 | NT); "
                    f"median of {reps} per-call events"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp_decode, min_seconds=10.0, single_thread_seconds=4.0):
    """The oracle on this host, on the decode batch, repeated for >= min_seconds
    with up to 16 threads, then for >= single_thread_seconds on one thread."""
    import dataclasses

    import oracle
    import workloads as wl

    _, pages = wl.decode_workload(seed=0)
    sub = dataclasses.replace(inp_decode.geom, num_slots=inp_decode.num_seqs)
    loc = np.arange(inp_decode.num_seqs, dtype=np.int32)

    def run(threads, seconds):
        oracle.set_threads(threads)
        reps, t0 = 0, time.perf_counter()
        while True:
            work = pages.copy()
            oracle.gdn_layer(work, sub, inp_decode.cu_seqlens, loc, inp_decode.has_initial_state,
                             inp_decode.x, inp_decode.conv_w, inp_decode.conv_b,
                             inp_decode.alpha, inp_decode.beta)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        return reps, time.perf_counter() - t0, oracle.get_threads()

    reps, dt, cores = run(min(os.cpu_count() or 1, 16), min_seconds)
    reps1, dt1, _ = run(1, single_thread_seconds)
    nb = decode_bytes(inp_decode)
    return {"value": round(nb * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"the full decode batch (256 rows x 32 heads) x {reps} repetitions, "
                      f"{dt:.1f} s, fp64 C oracle with OpenMP over rows",
            "single_thread_value": round(nb * reps1 / dt1 / 1e9, 4),
            "single_thread_sample": f"{reps1} repetitions on 1 thread, {dt1:.1f} s"}


def cpu_baseline_prefill(threads=None, single_thread_seqs=4):
    """The oracle on the 8-sequence prefill workload: the whole workload once
    with OpenMP over sequences (8 sequences, so at most 8 threads work), then
    the shortest `single_thread_seqs` sequences on one thread; tokens/s."""
    import dataclasses

    import oracle
    import workloads as wl

    inp, img = wl.prefill_workload(seed=0)
    g = inp.geom
    threads = threads or min(os.cpu_count() or 1, 16)

    def run(sub, n_threads):
        oracle.set_threads(n_threads)
        work = img.copy()
        t0 = time.perf_counter()
        oracle.gdn_layer(work, g, sub.cu_seqlens, sub.state_indices, sub.has_initial_state,
                         sub.x, sub.conv_w, sub.conv_b, sub.alpha, sub.beta)
        return time.perf_counter() - t0, oracle.get_threads()

    dt, got = run(inp, threads)
    lens = np.diff(inp.cu_seqlens)
    pick = np.sort(np.argsort(lens, kind="stable")[:single_thread_seqs])
    rows = np.concatenate([np.arange(inp.cu_seqlens[i], inp.cu_seqlens[i + 1]) for i in pick])
    cu = np.zeros(len(pick) + 1, np.int32)
    cu[1:] = np.cumsum(lens[pick])
    sub = dataclasses.replace(inp, x=inp.x[rows], alpha=inp.alpha[rows], beta=inp.beta[rows],
                              cu_seqlens=cu, state_indices=inp.state_indices[pick],
                              has_initial_state=inp.has_initial_state[pick])
    dt1, _ = run(sub, 1)
    return {"value": round(inp.total_tokens / dt, 1), "unit": "tokens/s",
            "cores": min(got, inp.num_seqs), "kind": "oracle", "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "sample": f"the whole 8-sequence prefill ({inp.total_tokens} tokens, 16 heads) once, "
                      f"{dt:.1f} s, fp64 C oracle with OpenMP over sequences ({got} threads "
                      f"offered, one per sequence busy)",
            "single_thread_value": round(sub.total_tokens / dt1, 1),
            "single_thread_sample": f"the {len(pick)} shortest sequences ({sub.total_tokens} "
                                    f"tokens) on 1 thread, {dt1:.1f} s"}


def cpu_baseline_restore(n_layers=11):
    """The oracle's restore of the 48-layer workload's 64 ops on a bounded
    sample of the stack: its first `n_layers` layers (9 GDN layers, every 4th
    attention-only), each a distinct host image of the touched pages, so that
    every page copy streams from memory; GB/s of the algorithmic bytes of the
    sample (the same bytes per GDN layer as the GPU restore)."""
    import dataclasses

    import oracle
    import workloads as wl

    g, linear, ops = wl.restore_workload(seed=0)
    linear = linear[:n_layers]
    hits = ops[:, 1] >= 0
    touched = np.unique(np.concatenate([ops[:, 0], ops[hits, 1]]))
    remap = {int(s_): i for i, s_ in enumerate(touched)}
    small = dataclasses.replace(g, num_slots=len(touched))
    ops_small = np.array([[remap[int(d)], remap[int(s_)] if s_ >= 0 else -1, r]
                          for d, s_, r in ops], np.int32)
    rng = np.random.default_rng(0)
    layers = [rng.integers(0, 256, (small.num_slots, g.page_stride), dtype=np.uint8)
              if lin else None for lin in linear]
    hs = np.ones(len(ops), np.uint8)
    oracle.restore(layers, small, ops_small, hs)  # first touch of the pages
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.restore(layers, small, ops_small, hs)
        reps += 1
        if time.perf_counter() - t0 >= 3.0:
            break
    dt = time.perf_counter() - t0
    nbytes = 2 * int(hits.sum()) * int(linear.sum()) * (g.ssm_region_bytes + g.conv_region_bytes)
    return {"value": round(nbytes * reps / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"the restore of the 64 ops ({int(hits.sum())} hits) over the stack's "
                      f"first {len(linear)} layers ({int(linear.sum())} GDN layers, distinct "
                      f"host images of the touched pages), {reps} repetitions, {dt:.1f} s, "
                      "plain C memcpy per (op, layer) region on one thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-restore", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (3 times), the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--only", choices=["prefill", "prefill32", "ceilings", "restore"],
                    help="run one secondary leg alone and print its figures (for counter "
                         "passes under rocprofv3); no bench line")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py measures one GPU only: the slot-state path has no cross-GPU step "
              "(each data-parallel rank owns its own pool); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import hybrid_linear_attention_slot_amd as gdn
    gdn.lib()

    if a.calibrate:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if a.only:
        if a.only == "prefill":
            pinp, ppc, _ = bench_prefill(a.steps, a.warmup, with_checkpoints=False)
            part = {"prefill_ms_p50": round(ppc["p50"], 4), "tokens": pinp.total_tokens}
        elif a.only == "prefill32":
            part = bench_prefill_32heads(a.steps, a.warmup)
        elif a.only == "restore":
            rms, rbytes, _, _, _, gs = bench_restore(a.steps, a.warmup)
            part = {"restore_ms_p50": round(rms, 4), "restore_gb_per_s": round(rbytes / (rms * 1e-3) / 1e9, 2),
                    "gather_gb_per_s": gs["gather"]["gb_per_s"], "scatter_gb_per_s": gs["scatter"]["gb_per_s"]}
        else:
            part = bench_ceilings()
        print(json.dumps({"only": a.only, **part}), flush=True)
        return
    inp, ms, nbytes, dpc = bench_decode(a.steps, a.warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    _, ms_pad, nbytes_pad, _ = bench_decode(a.steps, a.warmup, extra_pad=4096)
    torch.cuda.empty_cache()
    pinp, ppc, pms_ck = bench_prefill(a.steps, a.warmup)
    pms = ppc["p50"]
    pflops = prefill_flops(pinp) / (pms * 1e-3) / 1e12
    prefill = {"tokens_per_s": round(pinp.total_tokens / (pms * 1e-3), 1),
               "ms_per_call": round(pms, 4),
               "ms_p10_p90": [round(ppc["p10"], 4), round(ppc["p90"], 4)],
               "tokens": pinp.total_tokens,
               "max_seqlen": pinp.max_seqlen,
               "us_per_token_critical_path": round(pms * 1e3 / pinp.max_seqlen, 4),
               "gb_per_s": round(prefill_bytes(pinp) / (pms * 1e-3) / 1e9, 2),
               "tflops": round(pflops, 2),
               "frac_of_fp32_vector_peak": round(pflops / FP32_VECTOR_PEAK_TFLOPS, 4),
               "frac_of_fp32_nonpacked_peak": round(pflops / FP32_NONPACKED_PEAK_TFLOPS, 4),
               "arithmetic": "chunked delta rule (16-token chunks); products over the key "
                             "dimension and the chunk's tokens as three bf16 MFMA products "
                             "per fp32 product (hi*hi + hi*lo + lo*hi), fp32 accumulation; "
                             "flops above are the recurrence's algorithmic fp32 flops",
               "workload": "8 seqs, lengths U{512..4096}, 16 v-heads/8 k-heads, 128x128 fp32, "
                           "4 warm + 4 cold",
               "ms_per_call_with_checkpoints": round(pms_ck, 4),
               "checkpoints": "each sequence's state at its last 256-token boundary emitted "
                              "into a spare slot (gdn_prefill_varlen_checkpoint)",
               "timing": "median of per-call HIP event pairs"}
    prefill["heads_32"] = bench_prefill_32heads(a.steps, a.warmup)
    restore = None
    if not a.no_restore:
        rms, rbytes, hits, nlin, snap, gs = bench_restore(a.steps, a.warmup)
        restore = {"gb_per_s": round(rbytes / (rms * 1e-3) / 1e9, 2), "ms_per_call": round(rms, 4),
                   "bytes": rbytes, "hits": hits, "gdn_layers": nlin,
                   "frac_of_hbm_peak": round(rbytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "timing": "median of per-call HIP event pairs",
                   "gather_scatter": gs,
                   "snapshot_one_slot": snap}
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "per_launch_us": {k: round(v * 1e3, 2) for k, v in dpc.items()},
        "decode_4k_padded_pages": {"gb_per_s": round(nbytes_pad / (ms_pad * 1e-3) / 1e9, 2),
                                   "ms_per_step": round(ms_pad, 5),
                                   "note": "same step, 4 KiB of padding after every payload"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode step: 256 rows x 1 token, 32 v-heads / 16 k-heads, "
                               "128x128 fp32 state, conv 8192 bf16 x 4 taps, 1024-slot pool, "
                               "4 KiB-padded pages, 90% warm",
                   "rows": inp.num_seqs, "warm_rows": int(inp.has_initial_state.sum()),
                   "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(DECODE_PROFILE, DECODE_SOURCES)},
        "prefill": prefill,
        "restore": restore,
    }
    line["copy_baseline"] = bench_copy()
    ceil = bench_ceilings()
    ceil["decode_frac_of_rmw"] = round(gbs / ceil["rmw_gb_per_s"], 4)
    if restore is not None:
        restore["frac_of_copy_ceiling"] = round(restore["gb_per_s"] / ceil["copy_gb_per_s"], 4)
        for k in ("gather", "scatter"):
            gsk = restore["gather_scatter"][k]
            gsk["frac_of_copy_ceiling"] = round(gsk["gb_per_s"] / ceil["copy_gb_per_s"], 4)
    line["hbm_ceilings"] = ceil
    line["slot_manager"] = bench_slot_manager()
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp)
        prefill["cpu_baseline"] = cpu_baseline_prefill()
        if restore is not None:
            restore["cpu_baseline"] = cpu_baseline_restore()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
